// C ABI of libmfattn: argument checks, per-device state (workspace, cos/sin
// tables, status flag) and the launch sequence of the packed attention path:
//   meta_kernel      metadata check, padded offsets, longest-first tile table
//   rope_pack_kernel 2D RoPE on q, k into the padded workspace (+ V transpose)
//   attn_fwd_*       per-sample flash-style attention
// Nothing here synchronizes except mf_get_device_error / mf_get_workspace_error,
// the first-use allocations of the library-owned state, and the debug mode
// (MF_DEBUG=1 in the environment: every stage is followed by a stream
// synchronization and a check of the launch, of device faults and of the
// device flags, so a failure is reported by the call that caused it, naming
// the stage). Every stage is bracketed by a roctx range ("mf <kernel>"), which
// rocprofv3 --marker-trace records next to the kernels.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "mf_attn.h"
#include "mf_common.h"
#include "rope_math.h"

namespace mf {
hipError_t launch_meta(const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                       const int32_t* cu_in, int32_t n, int64_t tokens, char* ws, const WsLayout& l,
                       hipStream_t s);
hipError_t launch_build_metadata(const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                                 int32_t n, int64_t tokens, int32_t* cu_out, int32_t* pos, int32_t* seg_id,
                                 int32_t* status, hipStream_t s);
hipError_t launch_rope_pack(const void* q, const void* k, const void* v, const int32_t* grid_hw,
                            const int32_t* text_len, const char* ws, const WsLayout& l,
                            const float2* cs, const Rope3* r3, int32_t heads, int32_t head_dim, const Strides& st,
                            hipStream_t s);
hipError_t launch_prologue_bf16(const void* k, int64_t k_st, int64_t k_sh, const void* v, int64_t v_st, int64_t v_sh,
                                const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                                const int32_t* cu_in, int32_t n_seg, int64_t tokens, char* ws, const WsLayout& l,
                                const float2* cs, const Rope3* r3, int32_t heads, int32_t head_dim, bool fused,
                                hipStream_t s);
hipError_t launch_rope(const void* x, void* y, const int32_t* pos, int64_t tokens, int32_t heads,
                       int32_t head_dim, bool bf16, const float2* cs, const Rope3* r3, int32_t* status,
                       hipStream_t s);
hipError_t launch_attn_fwd(char* ws, const WsLayout& l, const void* q, const int32_t* grid_hw,
                           const int32_t* text_len, const float2* cs, const Rope3* r3, void* out, float* lse,
                           int64_t tokens, int32_t heads, int32_t head_dim, bool bf16, float scale, int32_t ncu,
                           const Strides& st, hipStream_t s);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const int32_t* grid_hw, const int32_t* text_len,
                           const float2* cs, const Rope3* r3, char* ws, const BwdLayout& l, void* dq, void* dk,
                           void* dv, int64_t tokens, int32_t heads, int32_t head_dim, float scale, int32_t ncu,
                           int32_t ncu_q, hipStream_t s, hipEvent_t const* ev);
hipError_t launch_qkv_fold(const void* w_txt, const void* w_img, const float* g_txt, const float* g_img,
                           int32_t hidden, int32_t out_features, void* out, hipStream_t s);
hipError_t launch_qkv(const void* x, const void* w, const int32_t* cu, const int32_t* grid_hw, const int32_t* text_len,
                      const int32_t* frames, int32_t n_seg, int64_t tokens, int32_t hidden, int32_t hd, float eps,
                      char* ws, void* q, void* k, void* v, int32_t ncu, hipStream_t s, hipEvent_t const* ev);
size_t qkv_workspace_bytes(int64_t tokens, int32_t n_seg, int32_t hidden);
hipError_t launch_pack(bool unpack, int32_t n_tensors, const void* const* src0, const void* const* src1,
                       void* const* dst0, void* const* dst1, const int32_t* cu, const int32_t* grid_hw,
                       const int32_t* text_len, const int32_t* frames, int32_t n_seg, int64_t tokens,
                       int64_t text_tokens, int64_t row_bytes, int32_t ncu, int32_t* status, hipStream_t s);
hipError_t launch_cfg_euler(float* z, const void* v, const int32_t* cu, const int32_t* grid_hw,
                            const int32_t* text_len, int32_t n_seg, int64_t total_tokens,
                            const int32_t* cond_seg, const int32_t* uncond_seg, int32_t n_img,
                            int64_t image_tokens, int32_t channels, bool bf16, float guidance, float dt,
                            int32_t* status, hipStream_t s);
}  // namespace mf

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// roctx range around the launches of one stage (host-side enqueue; the
// profiler correlates it with the kernels it enqueues).
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

bool debug_mode() {
  static const bool on = [] {
    const char* e = std::getenv("MF_DEBUG");
    return e && e[0] == '1';
  }();
  return on;
}

// Debug mode only: waits for the stream, then reports a failed launch, a
// device fault, or a set device flag (a workspace header's flag or the sticky
// status word; `clear` resets a status word once reported) as the error of
// this call. Outside debug mode it does nothing.
int debug_stage(hipStream_t s, const char* stage, const int32_t* flag = nullptr, bool clear = false) {
  if (!debug_mode()) return MF_OK;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MF_ERR_HIP, "%s: launch: %s", stage, hipGetErrorString(e));
  if ((e = hipStreamSynchronize(s)) != hipSuccess)
    return fail(MF_ERR_HIP, "%s: hipStreamSynchronize: %s", stage, hipGetErrorString(e));
  if (!flag) return MF_OK;
  int32_t v = 0;
  if ((e = hipMemcpy(&v, flag, 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return fail(MF_ERR_HIP, "%s: reading the device flag: %s", stage, hipGetErrorString(e));
  if (v && clear && (e = hipMemset(const_cast<int32_t*>(flag), 0, 4)) != hipSuccess)
    return fail(MF_ERR_HIP, "%s: clearing the device flag: %s", stage, hipGetErrorString(e));
  if (v) return fail(MF_ERR_METADATA, "%s: device check failed (flags 0x%x)", stage, unsigned(v));
  return MF_OK;
}

const int32_t* ws_flag(const char* ws) { return reinterpret_cast<const int32_t*>(ws); }  // WsHeader::flag

// Stream order of the calls that share one library workspace: the stream of
// the last call and an event recorded after its kernels.
struct WsOrder {
  hipEvent_t done = nullptr;
  hipStream_t last = nullptr;
  bool valid = false;
};

struct DeviceState {
  int32_t* status = nullptr;  // sticky FLAG_* of the standalone metadata / RoPE / sampler calls
  WsOrder ord_ws, ord_bws, ord_qws;  // order of the calls on ws, bws, qws
  char* ws = nullptr;         // library workspace of mf_attn_packed
  size_t ws_bytes = 0;
  char* bws = nullptr;        // library workspace of mf_attn_packed_bwd
  size_t bws_bytes = 0;
  char* qws = nullptr;        // library workspace of mf_qkv_rmsnorm
  size_t qws_bytes = 0;
  int32_t ncu = -1;           // compute units for the forward's split plan (0: splitting off); -1 unknown
  char* scratch = nullptr;    // this device's copy of the static scratch array (mf_attn_packed_noalloc)
  const float2* scratch_tables = nullptr;  // its copy of the static 2D cos/sin tables (d = 128, then d = 64)
  // (head_dim, theta bits, row channels, column channels) -> cos/sin table;
  // row channels -1 marks the 2D table
  std::map<std::tuple<int, uint32_t, int, int>, float2*> tables;
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;

int current_device(int* dev) {
  const hipError_t e = hipGetDevice(dev);
  return e == hipSuccess ? MF_OK : hip_fail(e, "hipGetDevice");
}

// Compute units of the device, for the forward's split of a partly filled
// last round (MF_ATTN_SPLIT=0 in the environment turns the split off).
// Caller holds g_mu.
int ensure_cus(DeviceState& st, int dev, int32_t* ncu) {
  if (st.ncu < 0) {
    int v = 0;
    const hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
    const char* off = std::getenv("MF_ATTN_SPLIT");
    st.ncu = off && off[0] == '0' ? 0 : v;
  }
  *ncu = st.ncu;
  return MF_OK;
}

// Caller holds g_mu.
int ensure_status(DeviceState& st) {
  if (st.status) return MF_OK;
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, 256);
  if (e != hipSuccess) return fail(MF_ERR_OOM, "status buffer: %s", hipGetErrorString(e));
  e = hipMemset(p, 0, 256);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return hip_fail(e, "hipMemset(status)");
  }
  st.status = static_cast<int32_t*>(p);
  return MF_OK;
}

int upload_table(DeviceState& st, std::tuple<int, uint32_t, int, int> key, const std::vector<float2>& host,
                 const float2** out) {
  void* d = nullptr;
  hipError_t e = hipMalloc(&d, host.size() * sizeof(float2));
  if (e != hipSuccess) return fail(MF_ERR_OOM, "rope table: %s", hipGetErrorString(e));
  e = hipMemcpy(d, host.data(), host.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(d);
    return hip_fail(e, "hipMemcpy(rope table)");
  }
  st.tables[key] = static_cast<float2*>(d);
  *out = static_cast<float2*>(d);
  return MF_OK;
}

// 2D cos/sin table [ROPE_PMAX][head_dim/4]: entry (p, j) = (cos, sin) of
// p * theta^(-2j/(head_dim/2)), evaluated in double and rounded to float.
std::vector<float2> table2d_host(int head_dim, float theta) {
  const int nf = head_dim / 4;
  std::vector<float2> host(size_t(mf::ROPE_PMAX) * nf);
  for (int p = 0; p < mf::ROPE_PMAX; ++p) {
    for (int j = 0; j < nf; ++j) {
      const double w = std::pow(double(theta), -2.0 * j / (head_dim / 2));
      const double ang = double(p) * w;
      host[size_t(p) * nf + j] = make_float2(float(std::cos(ang)), float(std::sin(ang)));
    }
  }
  return host;
}

// The 2D table of mf_attn_packed for this head_dim, created on first use.
// Caller holds g_mu.
int ensure_table(DeviceState& st, int head_dim, float theta, const float2** out) {
  uint32_t tb;
  std::memcpy(&tb, &theta, 4);
  const auto key = std::make_tuple(head_dim, tb, -1, -1);
  auto it = st.tables.find(key);
  if (it != st.tables.end()) {
    *out = it->second;
    return MF_OK;
  }
  return upload_table(st, key, table2d_host(head_dim, theta), out);
}

// Frame-aware cos/sin table [ROPE_PMAX][head_dim/2] for the channel split
// (row, col, head_dim - row - col): pair k of block a (channels m_a, local
// index j) has frequency theta^(-2j/m_a); entry (p, k) = (cos, sin) of p times
// it, evaluated in double. Caller holds g_mu.
int ensure_table3(DeviceState& st, int head_dim, float theta, int s_row, int s_col, const float2** out) {
  uint32_t tb;
  std::memcpy(&tb, &theta, 4);
  const auto key = std::make_tuple(head_dim, tb, s_row, s_col);
  auto it = st.tables.find(key);
  if (it != st.tables.end()) {
    *out = it->second;
    return MF_OK;
  }
  const int np = head_dim / 2;
  const int bound[3] = {s_row / 2, (s_row + s_col) / 2, np};
  const int m[3] = {s_row, s_col, head_dim - s_row - s_col};
  std::vector<float2> host(size_t(mf::ROPE_PMAX) * np);
  for (int k = 0; k < np; ++k) {
    const int a = k < bound[0] ? 0 : (k < bound[1] ? 1 : 2);
    const int j = k - (a == 0 ? 0 : bound[a - 1]);
    const double w = std::pow(double(theta), -2.0 * j / m[a]);
    for (int p = 0; p < mf::ROPE_PMAX; ++p) {
      const double ang = double(p) * w;
      host[size_t(p) * np + k] = make_float2(float(std::cos(ang)), float(std::sin(ang)));
    }
  }
  return upload_table(st, key, host, out);
}

int check_split(int32_t head_dim, int32_t s_row, int32_t s_col, int32_t s_frame) {
  if (s_row < 0 || s_col < 0 || s_frame < 0 || (s_row | s_col | s_frame) & 1 ||
      int64_t(s_row) + s_col + s_frame != head_dim)
    return fail(MF_ERR_INVALID_ARG, "rope split (%d, %d, %d) must be even, >= 0 and sum to head_dim=%d", s_row,
                s_col, s_frame, head_dim);
  return MF_OK;
}

// Grows a library-owned workspace (buf, have) to at least `bytes`; a new
// buffer starts with a zeroed header.
int ensure_buffer(char*& buf, size_t& have, size_t bytes) {
  if (have >= bytes) return MF_OK;
  const char* f = std::getenv("MF_FAULT_OOM");
  if (f && f[0] == '1') return fail(MF_ERR_OOM, "workspace of %zu bytes: injected failure", bytes);
  if (buf) {
    // hipFree waits for the device, so no enqueued call still uses the old buffer.
    const hipError_t e = hipFree(buf);
    buf = nullptr;
    have = 0;
    if (e != hipSuccess) return hip_fail(e, "hipFree(workspace)");
  }
  void* p = nullptr;
  const hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MF_ERR_OOM, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
  }
  const hipError_t z = hipMemset(p, 0, sizeof(mf::WsHeader));
  if (z != hipSuccess) {
    (void)hipFree(p);
    return hip_fail(z, "hipMemset(workspace header)");
  }
  buf = static_cast<char*>(p);
  have = bytes;
  return MF_OK;
}

int ensure_workspace(DeviceState& st, size_t bytes) { return ensure_buffer(st.ws, st.ws_bytes, bytes); }

// Runs launch() (which enqueues a call's kernels on stream s, all using one
// library workspace) after the previous call on that workspace: when that
// call was enqueued on another stream, s first waits (on the device) for the
// event recorded after it. Calls enqueued while s is being captured into a
// graph are not ordered this way (a captured graph cannot wait on an event
// recorded outside it), and the next call does not wait for them; a failed
// capture-status query counts as capturing. The event only orders work on
// this device, so it is recorded without the system-scope fence (which would
// write the L2 caches back for host visibility after every call). Caller
// holds g_mu.
template <typename F>
int ordered(WsOrder& o, hipStream_t s, F&& launch) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  bool capturing = true;
  if (hipStreamIsCapturing(s, &cs) == hipSuccess) capturing = cs != hipStreamCaptureStatusNone;
  else (void)hipGetLastError();
  hipError_t e;
  if (!capturing && o.valid && o.last != s && (e = hipStreamWaitEvent(s, o.done, 0)) != hipSuccess)
    return hip_fail(e, "hipStreamWaitEvent (workspace order)");
  const int rc = launch();
  if (capturing) {
    o.valid = false;
    return rc;
  }
  if (!o.done && (e = hipEventCreateWithFlags(&o.done, hipEventDisableTiming | hipEventDisableSystemFence)) != hipSuccess) {
    o.done = nullptr;
    o.valid = false;
    return rc ? rc : hip_fail(e, "hipEventCreateWithFlags (workspace order)");
  }
  if ((e = hipEventRecord(o.done, s)) != hipSuccess) {
    o.valid = false;
    return rc ? rc : hip_fail(e, "hipEventRecord (workspace order)");
  }
  o.last = s;
  o.valid = true;
  return rc;
}

int elem_bytes(int32_t dtype) { return dtype == MF_BF16 ? 2 : dtype == MF_F32 ? 4 : 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checks of the attention entry points that do not depend on the tensors'
// layout: null pointers, sizes, dtype.
int check_attn_scalars(const void* q, const void* k, const void* v, const int32_t* cu,
                       const int32_t* grid_hw, const int32_t* text_len, const void* out,
                       int32_t n_seg, int64_t tokens, int32_t heads, int32_t head_dim,
                       int32_t dtype) {
  if (!q || !k || !v || !cu || !grid_hw || !text_len || !out)
    return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  if (n_seg < 1 || n_seg > MF_MAX_SEGMENTS)
    return fail(MF_ERR_INVALID_ARG, "n_seg=%d outside [1, %d]", n_seg, MF_MAX_SEGMENTS);
  if (tokens < 1 || tokens >= (int64_t(1) << 31))
    return fail(MF_ERR_INVALID_ARG, "total_tokens=%lld outside [1, 2^31)", (long long)tokens);
  if (heads < 1 || heads > 256) return fail(MF_ERR_INVALID_ARG, "heads=%d outside [1, 256]", heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(MF_ERR_UNSUPPORTED, "head_dim=%d (supported: 64, 128)", head_dim);
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(MF_ERR_UNSUPPORTED, "dtype=%d (supported: MF_BF16, MF_F32)", dtype);
  const mf::WsLayout l = mf::ws_layout(tokens, heads, head_dim, eb, n_seg);
  if (int64_t(heads) * l.rows * head_dim >= (int64_t(1) << 40) || l.n_tiles * heads >= (int64_t(1) << 31))
    return fail(MF_ERR_UNSUPPORTED, "problem too large");
  return MF_OK;
}

// All checks of the attention entry points on contiguous [T][heads][d] tensors.
int check_attn_args(const void* q, const void* k, const void* v, const int32_t* cu,
                    const int32_t* grid_hw, const int32_t* text_len, const void* out,
                    int32_t n_seg, int64_t tokens, int32_t heads, int32_t head_dim,
                    int32_t dtype) {
  const int rc = check_attn_scalars(q, k, v, cu, grid_hw, text_len, out, n_seg, tokens, heads, head_dim, dtype);
  if (rc) return rc;
  const size_t tb = size_t(tokens) * heads * head_dim * elem_bytes(dtype);
  if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb))
    return fail(MF_ERR_INVALID_ARG, "out overlaps q, k or v");
  if (overlaps(out, tb, cu, size_t(n_seg + 1) * 4) || overlaps(out, tb, grid_hw, size_t(n_seg) * 8) ||
      overlaps(out, tb, text_len, size_t(n_seg) * 4))
    return fail(MF_ERR_INVALID_ARG, "out overlaps the metadata");
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if (mis & 15) return fail(MF_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  return MF_OK;
}

int run_attn(const void* q, const void* k, const void* v, const int32_t* cu, const int32_t* grid_hw,
             const int32_t* text_len, void* out, int32_t n_seg, int64_t tokens, int32_t heads,
             int32_t head_dim, int32_t dtype, char* ws, const float2* cs, int32_t ncu, hipStream_t s,
             hipEvent_t const* ev = nullptr, float* lse = nullptr, const int32_t* frames = nullptr,
             const mf::Rope3* r3 = nullptr, bool with_parts = true, const mf::Strides* strides = nullptr) {
  const bool bf16 = dtype == MF_BF16;
  const mf::Strides st = strides ? *strides : mf::contiguous_strides(heads, head_dim);
  const mf::WsLayout l = mf::ws_layout(tokens, heads, head_dim, elem_bytes(dtype), n_seg, with_parts);
  if (!with_parts) ncu = 0;  // no partial-result slots: never split
  hipError_t e;
  int rc;
  // bf16 batches of at most 64 samples: the prologue derives the metadata
  // itself (one launch less); otherwise the metadata kernel runs first.
  const bool fused = bf16 && n_seg <= 64;
  if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (!fused) {
    {
      Range r("mf meta_kernel");
      e = mf::launch_meta(grid_hw, text_len, frames, cu, n_seg, tokens, ws, l, s);
    }
    if (e != hipSuccess) return hip_fail(e, "meta_kernel launch");
    if ((rc = debug_stage(s, "meta_kernel", ws_flag(ws)))) return rc;
  }
  if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  {
    Range r("mf rope prologue");
    if (bf16) {
      e = mf::launch_prologue_bf16(k, st.k_st, st.k_sh, v, st.v_st, st.v_sh, grid_hw, text_len, frames, cu, n_seg,
                                   tokens, ws, l, cs, r3, heads, head_dim, fused, s);
    } else {
      e = mf::launch_rope_pack(q, k, v, grid_hw, text_len, ws, l, cs, r3, heads, head_dim, st, s);
    }
  }
  if (e != hipSuccess) return hip_fail(e, "rope prologue launch");
  if ((rc = debug_stage(s, fused ? "metadata + rope prologue" : "rope prologue", fused ? ws_flag(ws) : nullptr)))
    return rc;
  if (ev && (e = hipEventRecord(ev[2], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  {
    Range r("mf attn_fwd");
    e = mf::launch_attn_fwd(ws, l, q, grid_hw, text_len, cs, r3, out, lse, tokens, heads, head_dim, bf16,
                            float(1.0 / std::sqrt(double(head_dim))),
                            mf::split_possible(tokens, n_seg) ? ncu : 0, st, s);
  }
  if (e != hipSuccess) return hip_fail(e, "attn_fwd launch");
  if ((rc = debug_stage(s, "attn_fwd"))) return rc;
  if (ev && (e = hipEventRecord(ev[3], s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return MF_OK;
}

}  // namespace

extern "C" {

int mf_version(void) { return 100; }

const char* mf_last_error(void) { return g_err.c_str(); }

size_t mf_workspace_bytes(int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                          int32_t n_seg) {
  const int eb = elem_bytes(dtype);
  if (!eb || (head_dim != 64 && head_dim != 128) || heads < 1 || heads > 256 || n_seg < 1 ||
      n_seg > MF_MAX_SEGMENTS || total_tokens < 1 || total_tokens >= (int64_t(1) << 31))
    return 0;
  return size_t(mf::ws_layout(total_tokens, heads, head_dim, eb, n_seg).total);
}

int mf_attn_packed_profiled(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                            const int32_t* grid_hw, const int32_t* text_len, void* out,
                            int32_t n_seg, int64_t total_tokens, int32_t heads, int32_t head_dim,
                            int32_t dtype, hipEvent_t const* events, hipStream_t stream) {
  int rc = check_attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens, heads,
                           head_dim, dtype);
  if (rc) return rc;
  int dev;
  if ((rc = current_device(&dev))) return rc;
  const size_t need = mf_workspace_bytes(total_tokens, heads, head_dim, dtype, n_seg);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  const float2* cs = nullptr;
  int32_t ncu = 0;
  if ((rc = ensure_table(st, head_dim, MF_ROPE_THETA, &cs))) return rc;
  if ((rc = ensure_cus(st, dev, &ncu))) return rc;
  if ((rc = ensure_workspace(st, need))) return rc;
  return ordered(st.ord_ws, stream, [&] {
    return run_attn(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens, heads, head_dim, dtype,
                    st.ws, cs, ncu, stream, events);
  });
}

int mf_attn_packed(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                   const int32_t* grid_hw, const int32_t* text_len, void* out, int32_t n_seg,
                   int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                   hipStream_t stream) {
  return mf_attn_packed_profiled(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens,
                                 heads, head_dim, dtype, nullptr, stream);
}

int mf_attn_packed_ws(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                      const int32_t* grid_hw, const int32_t* text_len, void* out, int32_t n_seg,
                      int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens, heads,
                           head_dim, dtype);
  if (rc) return rc;
  if (!workspace) return fail(MF_ERR_INVALID_ARG, "null workspace");
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(MF_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t need = mf_workspace_bytes(total_tokens, heads, head_dim, dtype, n_seg);
  if (workspace_bytes < need)
    return fail(MF_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const size_t tb = size_t(total_tokens) * heads * head_dim * elem_bytes(dtype);
  if (overlaps(workspace, need, out, tb) || overlaps(workspace, need, q, tb) ||
      overlaps(workspace, need, k, tb) || overlaps(workspace, need, v, tb))
    return fail(MF_ERR_INVALID_ARG, "workspace overlaps q, k, v or out");
  int dev;
  if ((rc = current_device(&dev))) return rc;
  const float2* cs = nullptr;
  int32_t ncu = 0;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if ((rc = ensure_table(g_dev[dev], head_dim, MF_ROPE_THETA, &cs))) return rc;
    if ((rc = ensure_cus(g_dev[dev], dev, &ncu))) return rc;
  }
  return run_attn(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens, heads, head_dim,
                  dtype, static_cast<char*>(workspace), cs, ncu, stream);
}

}  // extern "C"

namespace {

// Forward with optional LSE; frames/split select the frame-aware RoPE.
int attn_impl(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, const int32_t* grid_hw,
              const int32_t* text_len, const int32_t* frames, const int32_t* split, void* out, float* lse,
              int32_t n_seg, int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
              hipStream_t stream) {
  int rc = check_attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens, heads,
                           head_dim, dtype);
  if (rc) return rc;
  if (split && (rc = check_split(head_dim, split[0], split[1], split[2]))) return rc;
  if (split && !frames) return fail(MF_ERR_INVALID_ARG, "null frames");
  const size_t tb = size_t(total_tokens) * heads * head_dim * elem_bytes(dtype);
  if (lse) {
    if (reinterpret_cast<uintptr_t>(lse) & 3) return fail(MF_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const size_t lb = size_t(total_tokens) * heads * 4;
    if (overlaps(lse, lb, out, tb) || overlaps(lse, lb, q, tb) || overlaps(lse, lb, k, tb) ||
        overlaps(lse, lb, v, tb))
      return fail(MF_ERR_INVALID_ARG, "lse overlaps q, k, v or out");
  }
  if (frames && overlaps(out, tb, frames, size_t(n_seg) * 4))
    return fail(MF_ERR_INVALID_ARG, "out overlaps frames");
  int dev;
  if ((rc = current_device(&dev))) return rc;
  const size_t need = mf_workspace_bytes(total_tokens, heads, head_dim, dtype, n_seg);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  const float2* cs = nullptr;
  mf::Rope3 r3{nullptr, 0, 0};
  if (split) {
    if ((rc = ensure_table3(st, head_dim, MF_ROPE_THETA, split[0], split[1], &r3.cs))) return rc;
    r3.b1 = split[0] / 2;
    r3.b2 = (split[0] + split[1]) / 2;
  } else if ((rc = ensure_table(st, head_dim, MF_ROPE_THETA, &cs))) {
    return rc;
  }
  int32_t ncu = 0;
  if ((rc = ensure_cus(st, dev, &ncu))) return rc;
  if ((rc = ensure_workspace(st, need))) return rc;
  return ordered(st.ord_ws, stream, [&] {
    return run_attn(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens, heads, head_dim, dtype,
                    st.ws, cs, ncu, stream, nullptr, lse, frames, split ? &r3 : nullptr);
  });
}

int bwd_launch(const void* q, const void* k, const void* v, const void* out, const void* d_out, const float* lse,
               const int32_t* cu_seqlens, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
               const mf::Rope3* r3, const float2* cs, void* dq, void* dk, void* dv, int32_t n_seg,
               int64_t total_tokens, int32_t heads, int32_t head_dim, char* bws, const mf::BwdLayout& l, int32_t ncu,
               int32_t ncu_q, hipEvent_t const* events, hipStream_t stream);

int bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* d_out, const float* lse,
             const int32_t* cu_seqlens, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
             const int32_t* split, void* dq, void* dk, void* dv, int32_t n_seg, int64_t total_tokens,
             int32_t heads, int32_t head_dim, int32_t dtype, hipEvent_t const* events, hipStream_t stream) {
  int rc = check_attn_args(q, k, v, cu_seqlens, grid_hw, text_len, dq, n_seg, total_tokens, heads,
                           head_dim, dtype);
  if (rc) return rc;
  if (dtype != MF_BF16) return fail(MF_ERR_UNSUPPORTED, "backward supports MF_BF16 only");
  if (!out || !d_out || !lse || !dk || !dv) return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  if (split && (rc = check_split(head_dim, split[0], split[1], split[2]))) return rc;
  if (split && !frames) return fail(MF_ERR_INVALID_ARG, "null frames");
  const size_t tb = size_t(total_tokens) * heads * head_dim * 2;
  const size_t lb = size_t(total_tokens) * heads * 4;
  const void* ins[6] = {q, k, v, out, d_out, lse};
  const size_t in_bytes[6] = {tb, tb, tb, tb, tb, lb};
  void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], tb, ins[j], in_bytes[j]))
        return fail(MF_ERR_INVALID_ARG, "a gradient output overlaps an input");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], tb, outs[j], tb)) return fail(MF_ERR_INVALID_ARG, "gradient outputs overlap");
    if (overlaps(outs[i], tb, cu_seqlens, size_t(n_seg + 1) * 4) ||
        overlaps(outs[i], tb, grid_hw, size_t(n_seg) * 8) || overlaps(outs[i], tb, text_len, size_t(n_seg) * 4) ||
        (frames && overlaps(outs[i], tb, frames, size_t(n_seg) * 4)))
      return fail(MF_ERR_INVALID_ARG, "a gradient output overlaps the metadata");
  }
  const uintptr_t mis = reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(d_out) |
                        reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
  if ((mis & 15) || (reinterpret_cast<uintptr_t>(lse) & 3))
    return fail(MF_ERR_INVALID_ARG, "out, d_out, dk, dv must be 16-byte aligned and lse 4-byte aligned");
  int dev;
  if ((rc = current_device(&dev))) return rc;
  const mf::BwdLayout l = mf::bwd_layout(total_tokens, heads, head_dim, n_seg);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  const float2* cs = nullptr;
  mf::Rope3 r3{nullptr, 0, 0};
  if (split) {
    if ((rc = ensure_table3(st, head_dim, MF_ROPE_THETA, split[0], split[1], &r3.cs))) return rc;
    r3.b1 = split[0] / 2;
    r3.b2 = (split[0] + split[1]) / 2;
  } else if ((rc = ensure_table(st, head_dim, MF_ROPE_THETA, &cs))) {
    return rc;
  }
  if ((rc = ensure_buffer(st.bws, st.bws_bytes, size_t(l.total)))) return rc;
  int32_t ncu = 0;
  if ((rc = ensure_cus(st, dev, &ncu))) return rc;
  // dQ units split with the forward's threshold, dK/dV units with the backward's.
  const int32_t ncu_q = mf::split_possible(total_tokens, n_seg) ? ncu : 0;
  if (!mf::split_possible(total_tokens, n_seg, mf::SPLIT_MIN_SAVED_BWD)) ncu = 0;
  return ordered(st.ord_bws, stream, [&] {
    return bwd_launch(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, frames, split ? &r3 : nullptr, cs,
                      dq, dk, dv, n_seg, total_tokens, heads, head_dim, st.bws, l, ncu, ncu_q, events, stream);
  });
}

// The backward's kernels on the library workspace bws (layout l).
int bwd_launch(const void* q, const void* k, const void* v, const void* out, const void* d_out, const float* lse,
               const int32_t* cu_seqlens, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
               const mf::Rope3* r3, const float2* cs, void* dq, void* dk, void* dv, int32_t n_seg,
               int64_t total_tokens, int32_t heads, int32_t head_dim, char* bws, const mf::BwdLayout& l, int32_t ncu,
               int32_t ncu_q, hipEvent_t const* events, hipStream_t stream) {
  int rc;
  hipError_t e;
  if (events && (e = hipEventRecord(events[0], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  {
    Range r("mf meta_kernel");
    e = mf::launch_meta(grid_hw, text_len, frames, cu_seqlens, n_seg, total_tokens, bws, l.m, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "meta_kernel launch");
  if ((rc = debug_stage(stream, "meta_kernel", ws_flag(bws)))) return rc;
  {
    Range r("mf attn_bwd");
    e = mf::launch_attn_bwd(q, k, v, out, d_out, lse, grid_hw, text_len, cs, r3, bws, l, dq, dk, dv, total_tokens,
                            heads, head_dim, float(1.0 / std::sqrt(double(head_dim))), ncu, ncu_q, stream,
                            events ? events + 1 : nullptr);
  }
  if (e != hipSuccess) return hip_fail(e, "backward kernels launch");
  if ((rc = debug_stage(stream, "backward kernels"))) return rc;
  if (events && (e = hipEventRecord(events[3], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return MF_OK;
}

int metadata_impl(int32_t n_seg, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                  int32_t* cu_seqlens_out, int32_t* pos_out, int32_t* seg_id_out, int64_t total_tokens,
                  hipStream_t stream) {
  if (!grid_hw || !text_len || !cu_seqlens_out || !pos_out || !seg_id_out)
    return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  if (n_seg < 1 || n_seg > MF_MAX_SEGMENTS)
    return fail(MF_ERR_INVALID_ARG, "n_seg=%d outside [1, %d]", n_seg, MF_MAX_SEGMENTS);
  if (total_tokens < 1 || total_tokens >= (int64_t(1) << 31))
    return fail(MF_ERR_INVALID_ARG, "total_tokens=%lld outside [1, 2^31)", (long long)total_tokens);
  int dev, rc;
  if ((rc = current_device(&dev))) return rc;
  int32_t* status;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if ((rc = ensure_status(g_dev[dev]))) return rc;
    status = g_dev[dev].status;
  }
  hipError_t e;
  {
    Range r("mf metadata");
    e = mf::launch_build_metadata(grid_hw, text_len, frames, n_seg, total_tokens, cu_seqlens_out, pos_out,
                                  seg_id_out, status, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "metadata kernels launch");
  return debug_stage(stream, "metadata kernels", status, true);
}

int rope_impl(const void* x_in, void* x_out, const int32_t* pos, const int32_t* split, int64_t total_tokens,
              int32_t heads, int32_t head_dim, int32_t dtype, float theta, hipStream_t stream) {
  if (!x_in || !x_out || !pos) return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  if (total_tokens < 1 || total_tokens >= (int64_t(1) << 31))
    return fail(MF_ERR_INVALID_ARG, "total_tokens=%lld outside [1, 2^31)", (long long)total_tokens);
  if (heads < 1 || heads > 256) return fail(MF_ERR_INVALID_ARG, "heads=%d outside [1, 256]", heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(MF_ERR_UNSUPPORTED, "head_dim=%d (supported: 64, 128)", head_dim);
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(MF_ERR_UNSUPPORTED, "dtype=%d", dtype);
  if (!(theta > 1.0f) || !std::isfinite(theta)) return fail(MF_ERR_INVALID_ARG, "theta must be > 1");
  int rc;
  if (split && (rc = check_split(head_dim, split[0], split[1], split[2]))) return rc;
  const size_t tb = size_t(total_tokens) * heads * head_dim * eb;
  if (x_in != x_out && overlaps(x_in, tb, x_out, tb))
    return fail(MF_ERR_INVALID_ARG, "x_in and x_out partially overlap");
  if ((reinterpret_cast<uintptr_t>(x_in) | reinterpret_cast<uintptr_t>(x_out)) & 15)
    return fail(MF_ERR_INVALID_ARG, "x_in and x_out must be 16-byte aligned");
  int dev;
  if ((rc = current_device(&dev))) return rc;
  const float2* cs = nullptr;
  mf::Rope3 r3{nullptr, 0, 0};
  int32_t* status;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& st = g_dev[dev];
    if ((rc = ensure_status(st))) return rc;
    if (split) {
      if ((rc = ensure_table3(st, head_dim, theta, split[0], split[1], &r3.cs))) return rc;
      r3.b1 = split[0] / 2;
      r3.b2 = (split[0] + split[1]) / 2;
    } else if ((rc = ensure_table(st, head_dim, theta, &cs))) {
      return rc;
    }
    status = st.status;
  }
  hipError_t e;
  {
    Range r("mf rope_kernel");
    e = mf::launch_rope(x_in, x_out, pos, total_tokens, heads, head_dim, dtype == MF_BF16, cs,
                        split ? &r3 : nullptr, status, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "rope_kernel launch");
  return debug_stage(stream, "rope_kernel", status, true);
}

}  // namespace

extern "C" {

int mf_attn_packed_lse(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                       const int32_t* grid_hw, const int32_t* text_len, void* out, float* lse,
                       int32_t n_seg, int64_t total_tokens, int32_t heads, int32_t head_dim,
                       int32_t dtype, hipStream_t stream) {
  if (!lse) return fail(MF_ERR_INVALID_ARG, "null lse");
  return attn_impl(q, k, v, cu_seqlens, grid_hw, text_len, nullptr, nullptr, out, lse, n_seg, total_tokens, heads,
                   head_dim, dtype, stream);
}

int mf_attn_packed_3d(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                      const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames, int32_t split_row,
                      int32_t split_col, int32_t split_frame, void* out, float* lse, int32_t n_seg,
                      int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  const int32_t split[3] = {split_row, split_col, split_frame};
  return attn_impl(q, k, v, cu_seqlens, grid_hw, text_len, frames, split, out, lse, n_seg, total_tokens, heads,
                   head_dim, dtype, stream);
}

int mf_attn_packed_3d_bwd(const void* q, const void* k, const void* v, const void* out, const void* d_out,
                          const float* lse, const int32_t* cu_seqlens, const int32_t* grid_hw,
                          const int32_t* text_len, const int32_t* frames, int32_t split_row, int32_t split_col,
                          int32_t split_frame, void* dq, void* dk, void* dv, int32_t n_seg, int64_t total_tokens,
                          int32_t heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  const int32_t split[3] = {split_row, split_col, split_frame};
  return bwd_impl(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, frames, split, dq, dk, dv, n_seg,
                  total_tokens, heads, head_dim, dtype, nullptr, stream);
}

size_t mf_bwd_workspace_bytes(int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t n_seg) {
  if ((head_dim != 64 && head_dim != 128) || heads < 1 || heads > 256 || n_seg < 1 ||
      n_seg > MF_MAX_SEGMENTS || total_tokens < 1 || total_tokens >= (int64_t(1) << 31))
    return 0;
  return size_t(mf::bwd_layout(total_tokens, heads, head_dim, n_seg).total);
}

int mf_attn_packed_bwd_profiled(const void* q, const void* k, const void* v, const void* out,
                                const void* d_out, const float* lse, const int32_t* cu_seqlens,
                                const int32_t* grid_hw, const int32_t* text_len, void* dq, void* dk,
                                void* dv, int32_t n_seg, int64_t total_tokens, int32_t heads,
                                int32_t head_dim, int32_t dtype, hipEvent_t const* events,
                                hipStream_t stream) {
  return bwd_impl(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, nullptr, nullptr, dq, dk, dv, n_seg,
                  total_tokens, heads, head_dim, dtype, events, stream);
}

int mf_attn_packed_bwd(const void* q, const void* k, const void* v, const void* out, const void* d_out,
                       const float* lse, const int32_t* cu_seqlens, const int32_t* grid_hw,
                       const int32_t* text_len, void* dq, void* dk, void* dv, int32_t n_seg,
                       int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                       hipStream_t stream) {
  return mf_attn_packed_bwd_profiled(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, dq, dk, dv,
                                     n_seg, total_tokens, heads, head_dim, dtype, nullptr, stream);
}

int mf_build_metadata(int32_t n_seg, const int32_t* grid_hw, const int32_t* text_len,
                      int32_t* cu_seqlens_out, int32_t* pos_out, int32_t* seg_id_out,
                      int64_t total_tokens, hipStream_t stream) {
  return metadata_impl(n_seg, grid_hw, text_len, nullptr, cu_seqlens_out, pos_out, seg_id_out, total_tokens,
                       stream);
}

int mf_build_metadata_3d(int32_t n_seg, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                         int32_t* cu_seqlens_out, int32_t* pos_out, int32_t* seg_id_out, int64_t total_tokens,
                         hipStream_t stream) {
  if (!frames) return fail(MF_ERR_INVALID_ARG, "null frames");
  return metadata_impl(n_seg, grid_hw, text_len, frames, cu_seqlens_out, pos_out, seg_id_out, total_tokens,
                       stream);
}

int mf_rope_2d(const void* x_in, void* x_out, const int32_t* pos, int64_t total_tokens,
               int32_t heads, int32_t head_dim, int32_t dtype, float theta, hipStream_t stream) {
  return rope_impl(x_in, x_out, pos, nullptr, total_tokens, heads, head_dim, dtype, theta, stream);
}

int mf_rope_3d(const void* x_in, void* x_out, const int32_t* pos, int64_t total_tokens, int32_t heads,
               int32_t head_dim, int32_t dtype, float theta, int32_t split_row, int32_t split_col,
               int32_t split_frame, hipStream_t stream) {
  const int32_t split[3] = {split_row, split_col, split_frame};
  return rope_impl(x_in, x_out, pos, split, total_tokens, heads, head_dim, dtype, theta, stream);
}

int mf_qkv_fold_weights(const void* w_txt, const void* w_img, const float* gamma_txt, const float* gamma_img,
                        int32_t hidden, int32_t heads, int32_t head_dim, void* w_out, hipStream_t stream) {
  if (!w_txt || !w_img || !gamma_txt || !gamma_img || !w_out) return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  if (hidden < 64 || hidden > 65536 || hidden % 64)
    return fail(MF_ERR_UNSUPPORTED, "hidden=%d (need a multiple of 64 in [64, 65536])", hidden);
  if (heads < 1 || head_dim < 1 || int64_t(heads) * head_dim % 256 || int64_t(heads) * head_dim > 65536)
    return fail(MF_ERR_UNSUPPORTED, "heads * head_dim = %lld (need a multiple of 256, at most 65536)",
                (long long)(int64_t(heads) * head_dim));
  const int32_t out_features = 3 * heads * head_dim;
  const size_t wb = size_t(out_features) * hidden * 2;
  if (overlaps(w_out, 2 * wb, w_txt, wb) || overlaps(w_out, 2 * wb, w_img, wb))
    return fail(MF_ERR_INVALID_ARG, "w_out overlaps an input weight");
  if ((reinterpret_cast<uintptr_t>(w_txt) | reinterpret_cast<uintptr_t>(w_img) | reinterpret_cast<uintptr_t>(w_out)) & 15)
    return fail(MF_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  const hipError_t e = mf::launch_qkv_fold(w_txt, w_img, gamma_txt, gamma_img, hidden, out_features, w_out, stream);
  return e == hipSuccess ? MF_OK : hip_fail(e, "qkv_fold_kernel launch");
}

int mf_qkv_rmsnorm_profiled(const void* x, const void* w_folded, const int32_t* cu_seqlens, const int32_t* grid_hw,
                            const int32_t* text_len, const int32_t* frames, int32_t n_seg, int64_t total_tokens,
                            int32_t hidden, int32_t heads, int32_t head_dim, float eps, void* q, void* k, void* v,
                            hipEvent_t const* events, hipStream_t stream) {
  if (!x || !w_folded || !cu_seqlens || !grid_hw || !text_len || !q || !k || !v)
    return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  if (n_seg < 1 || n_seg > MF_MAX_SEGMENTS)
    return fail(MF_ERR_INVALID_ARG, "n_seg=%d outside [1, %d]", n_seg, MF_MAX_SEGMENTS);
  if (total_tokens < 1 || total_tokens >= (int64_t(1) << 31))
    return fail(MF_ERR_INVALID_ARG, "total_tokens=%lld outside [1, 2^31)", (long long)total_tokens);
  if (hidden < 64 || hidden > 65536 || hidden % 64)
    return fail(MF_ERR_UNSUPPORTED, "hidden=%d (need a multiple of 64 in [64, 65536])", hidden);
  if (heads < 1 || head_dim < 1 || int64_t(heads) * head_dim % 256 || int64_t(heads) * head_dim > 65536)
    return fail(MF_ERR_UNSUPPORTED, "heads * head_dim = %lld (need a multiple of 256, at most 65536)",
                (long long)(int64_t(heads) * head_dim));
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(MF_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const int32_t hd = heads * head_dim;
  const size_t xb = size_t(total_tokens) * hidden * 2, ob = size_t(total_tokens) * hd * 2,
               wb = size_t(6) * hd * hidden * 2;
  void* outs[3] = {q, k, v};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], ob, x, xb) || overlaps(outs[i], ob, w_folded, wb))
      return fail(MF_ERR_INVALID_ARG, "q, k or v overlaps x or the weights");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], ob, outs[j], ob)) return fail(MF_ERR_INVALID_ARG, "q, k, v overlap");
  }
  const uintptr_t mis = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w_folded) |
                        reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v);
  if (mis & 15) return fail(MF_ERR_INVALID_ARG, "x, weights, q, k, v must be 16-byte aligned");
  int dev, rc;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  if ((rc = ensure_buffer(st.qws, st.qws_bytes, mf::qkv_workspace_bytes(total_tokens, n_seg, hidden)))) return rc;
  int32_t ncu = 0;
  if ((rc = ensure_cus(st, dev, &ncu))) return rc;
  return ordered(st.ord_qws, stream, [&] {
    hipError_t e;
    int rc2;
    if (events && (e = hipEventRecord(events[0], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    {
      Range r("mf qkv_rmsnorm");
      e = mf::launch_qkv(x, w_folded, cu_seqlens, grid_hw, text_len, frames, n_seg, total_tokens, hidden, hd, eps,
                         st.qws, q, k, v, ncu, stream, events ? events + 1 : nullptr);
    }
    if (e != hipSuccess) return hip_fail(e, "qkv kernels launch");
    if ((rc2 = debug_stage(stream, "qkv kernels", ws_flag(st.qws)))) return rc2;
    if (events && (e = hipEventRecord(events[2], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    return int(MF_OK);
  });
}

int mf_qkv_rmsnorm(const void* x, const void* w_folded, const int32_t* cu_seqlens, const int32_t* grid_hw,
                   const int32_t* text_len, const int32_t* frames, int32_t n_seg, int64_t total_tokens, int32_t hidden,
                   int32_t heads, int32_t head_dim, float eps, void* q, void* k, void* v, hipStream_t stream) {
  return mf_qkv_rmsnorm_profiled(x, w_folded, cu_seqlens, grid_hw, text_len, frames, n_seg, total_tokens, hidden,
                                 heads, head_dim, eps, q, k, v, nullptr, stream);
}

int mf_rf_cfg_euler_step(float* z, const void* v, const int32_t* cu_seqlens, const int32_t* grid_hw,
                         const int32_t* text_len, int32_t n_seg, int64_t total_tokens,
                         const int32_t* cond_seg, const int32_t* uncond_seg, int32_t n_img,
                         int64_t image_tokens, int32_t channels, int32_t dtype, float guidance,
                         float dt, hipStream_t stream) {
  if (!z || !v || !cu_seqlens || !grid_hw || !text_len || !cond_seg || !uncond_seg)
    return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  if (n_seg < 1 || n_seg > MF_MAX_SEGMENTS)
    return fail(MF_ERR_INVALID_ARG, "n_seg=%d outside [1, %d]", n_seg, MF_MAX_SEGMENTS);
  if (n_img < 1 || n_img > MF_MAX_SEGMENTS)
    return fail(MF_ERR_INVALID_ARG, "n_img=%d outside [1, %d]", n_img, MF_MAX_SEGMENTS);
  if (total_tokens < 1 || total_tokens >= (int64_t(1) << 31))
    return fail(MF_ERR_INVALID_ARG, "total_tokens=%lld outside [1, 2^31)", (long long)total_tokens);
  if (image_tokens < 1 || image_tokens >= (int64_t(1) << 31))
    return fail(MF_ERR_INVALID_ARG, "image_tokens=%lld outside [1, 2^31)", (long long)image_tokens);
  if (channels < 8 || channels > 4096 || channels % 8)
    return fail(MF_ERR_UNSUPPORTED, "channels=%d (need a multiple of 8 in [8, 4096])", channels);
  const int64_t chunks = image_tokens * (channels / 8);
  if (chunks >= (int64_t(1) << 31)) return fail(MF_ERR_INVALID_ARG, "image_tokens * channels / 8 >= 2^31");
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(MF_ERR_UNSUPPORTED, "dtype=%d", dtype);
  if (!std::isfinite(guidance) || !std::isfinite(dt))
    return fail(MF_ERR_INVALID_ARG, "guidance and dt must be finite");
  if ((reinterpret_cast<uintptr_t>(z) | reinterpret_cast<uintptr_t>(v)) & 15)
    return fail(MF_ERR_INVALID_ARG, "z and v must be 16-byte aligned");
  const size_t zb = size_t(image_tokens) * channels * 4, vb = size_t(total_tokens) * channels * eb;
  if (overlaps(z, zb, v, vb) || overlaps(z, zb, cu_seqlens, size_t(n_seg + 1) * 4) ||
      overlaps(z, zb, grid_hw, size_t(n_seg) * 8) || overlaps(z, zb, text_len, size_t(n_seg) * 4) ||
      overlaps(z, zb, cond_seg, size_t(n_img) * 4) || overlaps(z, zb, uncond_seg, size_t(n_img) * 4))
    return fail(MF_ERR_INVALID_ARG, "z overlaps another argument");
  int dev, rc;
  if ((rc = current_device(&dev))) return rc;
  int32_t* status;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& st = g_dev[dev];
    if ((rc = ensure_status(st))) return rc;
    status = st.status;
  }
  hipError_t e;
  {
    Range r("mf cfg_euler_kernel");
    e = mf::launch_cfg_euler(z, v, cu_seqlens, grid_hw, text_len, n_seg, total_tokens, cond_seg, uncond_seg, n_img,
                             image_tokens, channels, dtype == MF_BF16, guidance, dt, status, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "cfg_euler_kernel launch");
  return debug_stage(stream, "cfg_euler_kernel", status, true);
}

}  // extern "C"

namespace {

// Joint-layout pack (unpack == false: text/image streams -> joint rows) or
// unpack (joint rows -> streams) of n_tensors tensors in one launch.
int pack_impl(bool unpack, int32_t n_tensors, const void* const* a0, const void* const* a1, void* const* b0,
              void* const* b1, const int32_t* cu_seqlens, const int32_t* grid_hw, const int32_t* text_len,
              const int32_t* frames, int32_t n_seg, int64_t total_tokens, int64_t text_tokens, int32_t heads,
              int32_t head_dim, int32_t dtype, hipStream_t stream) {
  if (n_tensors < 1 || n_tensors > 4) return fail(MF_ERR_INVALID_ARG, "n_tensors=%d outside [1, 4]", n_tensors);
  if (!a0 || !b0 || (unpack ? !b1 : !a1) || !cu_seqlens || !grid_hw || !text_len)
    return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  if (n_seg < 1 || n_seg > MF_MAX_SEGMENTS)
    return fail(MF_ERR_INVALID_ARG, "n_seg=%d outside [1, %d]", n_seg, MF_MAX_SEGMENTS);
  if (total_tokens < 1 || total_tokens >= (int64_t(1) << 31))
    return fail(MF_ERR_INVALID_ARG, "total_tokens=%lld outside [1, 2^31)", (long long)total_tokens);
  if (text_tokens < 0 || text_tokens > total_tokens)
    return fail(MF_ERR_INVALID_ARG, "text_tokens=%lld outside [0, total_tokens]", (long long)text_tokens);
  if (heads < 1 || heads > 256) return fail(MF_ERR_INVALID_ARG, "heads=%d outside [1, 256]", heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(MF_ERR_UNSUPPORTED, "head_dim=%d (supported: 64, 128)", head_dim);
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(MF_ERR_UNSUPPORTED, "dtype=%d (supported: MF_BF16, MF_F32)", dtype);
  const int64_t row = int64_t(heads) * head_dim * eb;
  const int64_t image_tokens = total_tokens - text_tokens;
  // The joint tensors and the two streams of every tensor, with their sizes.
  const void* joint[4];
  const void* txt[4];
  const void* img[4];
  for (int i = 0; i < n_tensors; ++i) {
    joint[i] = unpack ? a0[i] : b0[i];
    txt[i] = unpack ? b0[i] : a0[i];
    img[i] = unpack ? b1[i] : a1[i];
    if (!joint[i] || (text_tokens > 0 && !txt[i]) || (image_tokens > 0 && !img[i]))
      return fail(MF_ERR_INVALID_ARG, "null tensor pointer (tensor %d)", i);
    if ((reinterpret_cast<uintptr_t>(joint[i]) | reinterpret_cast<uintptr_t>(txt[i]) |
         reinterpret_cast<uintptr_t>(img[i])) & 15)
      return fail(MF_ERR_INVALID_ARG, "tensor %d is not 16-byte aligned", i);
  }
  // Destinations must not overlap each other, any source or the metadata.
  std::vector<std::pair<const void*, size_t>> dst, src;
  for (int i = 0; i < n_tensors; ++i) {
    auto& d = unpack ? dst : src;
    auto& j = unpack ? src : dst;
    j.emplace_back(joint[i], size_t(total_tokens * row));
    if (text_tokens > 0) d.emplace_back(txt[i], size_t(text_tokens * row));
    if (image_tokens > 0) d.emplace_back(img[i], size_t(image_tokens * row));
  }
  src.emplace_back(cu_seqlens, size_t(n_seg + 1) * 4);
  src.emplace_back(grid_hw, size_t(n_seg) * 8);
  src.emplace_back(text_len, size_t(n_seg) * 4);
  if (frames) src.emplace_back(frames, size_t(n_seg) * 4);
  for (size_t i = 0; i < dst.size(); ++i) {
    for (const auto& x : src)
      if (overlaps(dst[i].first, dst[i].second, x.first, x.second))
        return fail(MF_ERR_INVALID_ARG, "an output overlaps an input or the metadata");
    for (size_t j = i + 1; j < dst.size(); ++j)
      if (overlaps(dst[i].first, dst[i].second, dst[j].first, dst[j].second))
        return fail(MF_ERR_INVALID_ARG, "outputs overlap");
  }
  int dev, rc;
  if ((rc = current_device(&dev))) return rc;
  int32_t* status;
  int32_t ncu = 0;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& st = g_dev[dev];
    if ((rc = ensure_status(st))) return rc;
    if ((rc = ensure_cus(st, dev, &ncu))) return rc;
    status = st.status;
  }
  hipError_t e;
  {
    Range r(unpack ? "mf unpack_joint" : "mf pack_joint");
    e = mf::launch_pack(unpack, n_tensors, a0, a1, b0, b1, cu_seqlens, grid_hw, text_len, frames, n_seg,
                        total_tokens, text_tokens, row, ncu, status, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "pack_kernel launch");
  return debug_stage(stream, unpack ? "unpack_joint" : "pack_joint", status, true);
}

}  // namespace

extern "C" {

int mf_pack_joint(int32_t n_tensors, const void* const* text, const void* const* image, void* const* joint,
                  const int32_t* cu_seqlens, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                  int32_t n_seg, int64_t total_tokens, int64_t text_tokens, int32_t heads, int32_t head_dim,
                  int32_t dtype, hipStream_t stream) {
  if (!text || !image || !joint) return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  return pack_impl(false, n_tensors, text, image, joint, nullptr, cu_seqlens, grid_hw, text_len, frames, n_seg,
                   total_tokens, text_tokens, heads, head_dim, dtype, stream);
}

int mf_unpack_joint(int32_t n_tensors, const void* const* joint, void* const* text, void* const* image,
                    const int32_t* cu_seqlens, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                    int32_t n_seg, int64_t total_tokens, int64_t text_tokens, int32_t heads, int32_t head_dim,
                    int32_t dtype, hipStream_t stream) {
  if (!text || !image || !joint) return fail(MF_ERR_INVALID_ARG, "null pointer argument");
  return pack_impl(true, n_tensors, joint, nullptr, text, image, cu_seqlens, grid_hw, text_len, frames, n_seg,
                   total_tokens, text_tokens, heads, head_dim, dtype, stream);
}

int mf_get_device_error(hipStream_t stream) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int dev, rc;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  int32_t flags = 0;
  if (st.status) {
    int32_t v = 0;
    if ((e = hipMemcpy(&v, st.status, 4, hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(status)");
    if (v && (e = hipMemset(st.status, 0, 4)) != hipSuccess) return hip_fail(e, "hipMemset(status)");
    flags |= v;
  }
  // Workspace headers (their flag is the first field): a failed check is
  // marked as reported; the next call on that workspace rewrites the header.
  for (char* w : {st.qws, st.ws, st.bws, st.scratch}) {
    if (!w) continue;
    int32_t f = 0;
    if ((e = hipMemcpy(&f, w, sizeof(f), hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(workspace header)");
    if (f == mf::FLAG_OK || f == mf::FLAG_REPORTED) continue;
    flags |= f;
    const int32_t reported = mf::FLAG_REPORTED;
    if ((e = hipMemcpy(w, &reported, sizeof(reported), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy(workspace header)");
  }
  if (flags) return fail(MF_ERR_METADATA, "device check failed (flags 0x%x)", unsigned(flags));
  return MF_OK;
}

int mf_get_workspace_error(const void* workspace, hipStream_t stream) {
  if (!workspace) return fail(MF_ERR_INVALID_ARG, "null workspace");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  mf::WsHeader hdr;
  if ((e = hipMemcpy(&hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy(workspace header)");
  if (hdr.flag) return fail(MF_ERR_METADATA, "device check failed (flags 0x%x)", unsigned(hdr.flag));
  return MF_OK;
}

}  // extern "C"

namespace {

// Byte span [first, last) touched by a strided tensor.
std::pair<uintptr_t, uintptr_t> tensor_span(const mf_tensor& t, int eb) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(t.data);
  const int64_t last = (int64_t(t.tokens) - 1) * t.stride_token + (int64_t(t.heads) - 1) * t.stride_head + t.head_dim;
  return {a, a + uintptr_t(last) * eb};
}

bool spans_overlap(std::pair<uintptr_t, uintptr_t> x, std::pair<uintptr_t, uintptr_t> y) {
  return x.first < y.second && y.first < x.second;
}

}  // namespace

extern "C" {

int mf_attn_packed_strided(const mf_tensor* q, const mf_tensor* k, const mf_tensor* v, const int32_t* cu_seqlens,
                           const int32_t* grid_hw, const int32_t* text_len, int32_t n_seg, const mf_tensor* out,
                           hipStream_t stream) {
  if (!q || !k || !v || !out) return fail(MF_ERR_INVALID_ARG, "null tensor descriptor");
  const mf_tensor* ts[4] = {q, k, v, out};
  for (const mf_tensor* t : ts) {
    if (t->dtype != q->dtype || t->tokens != q->tokens || t->heads != q->heads || t->head_dim != q->head_dim)
      return fail(MF_ERR_INVALID_ARG, "q, k, v and out must agree on dtype, tokens, heads and head_dim");
  }
  const int64_t T = q->tokens;
  const int32_t H = q->heads, D = q->head_dim;
  int rc = check_attn_scalars(q->data, k->data, v->data, cu_seqlens, grid_hw, text_len, out->data, n_seg, T, H, D,
                              q->dtype);
  if (rc) return rc;
  const int eb = elem_bytes(q->dtype);
  const int64_t align = 16 / eb;  // elements per 16-byte chunk
  for (const mf_tensor* t : ts) {
    if (t->stride_token < D || t->stride_head < D || t->stride_token % align || t->stride_head % align)
      return fail(MF_ERR_INVALID_ARG,
                  "strides (%lld, %lld) must be at least head_dim=%d and multiples of %lld elements",
                  (long long)t->stride_token, (long long)t->stride_head, D, (long long)align);
    if (reinterpret_cast<uintptr_t>(t->data) & 15) return fail(MF_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  }
  for (const mf_tensor* t : ts) {
    // extent below 2^60 elements (no overflow in the span arithmetic below)
    const int64_t lim = int64_t(1) << 60;
    if (t->stride_token > lim / T || t->stride_head > lim / H)
      return fail(MF_ERR_INVALID_ARG, "strides (%lld, %lld) too large", (long long)t->stride_token,
                  (long long)t->stride_head);
  }
  // out must be one-to-one: rows of a token (or of a head) must not interleave.
  const int64_t ost = out->stride_token, osh = out->stride_head;
  const bool token_major = osh >= D && ost >= (int64_t(H) - 1) * osh + D;
  const bool head_major = ost >= D && osh >= (T - 1) * ost + D;
  if (!token_major && !head_major)
    return fail(MF_ERR_INVALID_ARG, "out strides (%lld, %lld) let rows overlap", (long long)ost, (long long)osh);
  const auto os = tensor_span(*out, eb);
  for (const mf_tensor* t : {q, k, v})
    if (spans_overlap(os, tensor_span(*t, eb))) return fail(MF_ERR_INVALID_ARG, "out overlaps q, k or v");
  const std::pair<uintptr_t, uintptr_t> meta[3] = {
      {reinterpret_cast<uintptr_t>(cu_seqlens), reinterpret_cast<uintptr_t>(cu_seqlens) + size_t(n_seg + 1) * 4},
      {reinterpret_cast<uintptr_t>(grid_hw), reinterpret_cast<uintptr_t>(grid_hw) + size_t(n_seg) * 8},
      {reinterpret_cast<uintptr_t>(text_len), reinterpret_cast<uintptr_t>(text_len) + size_t(n_seg) * 4}};
  for (const auto& m : meta)
    if (spans_overlap(os, m)) return fail(MF_ERR_INVALID_ARG, "out overlaps the metadata");
  const mf::Strides st{q->stride_token, q->stride_head, k->stride_token, k->stride_head,
                       v->stride_token, v->stride_head, ost, osh};
  int dev;
  if ((rc = current_device(&dev))) return rc;
  const size_t need = mf_workspace_bytes(T, H, D, q->dtype, n_seg);
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& ds = g_dev[dev];
  const float2* cs = nullptr;
  int32_t ncu = 0;
  if ((rc = ensure_table(ds, D, MF_ROPE_THETA, &cs))) return rc;
  if ((rc = ensure_cus(ds, dev, &ncu))) return rc;
  if ((rc = ensure_workspace(ds, need))) return rc;
  return ordered(ds.ord_ws, stream, [&] {
    return run_attn(q->data, k->data, v->data, cu_seqlens, grid_hw, text_len, out->data, n_seg, T, H, D,
                    q->dtype, ds.ws, cs, ncu, stream, nullptr, nullptr, nullptr, nullptr, true, &st);
  });
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free forward for callers that cannot allocate device memory.
// The workspace is a file-scope static device array (every device the library
// runs on holds its own copy, allocated when this module is first used there
// and kept until the process ends); so are the 2D cos/sin tables. Host code
// never passes the arrays' names to a kernel (on the host they are stand-ins,
// not device addresses): the device addresses come from hipGetSymbolAddress,
// once per device, and only those are used.
namespace {

constexpr size_t NOALLOC_BYTES = size_t(MF_NOALLOC_SCRATCH_BYTES);
constexpr int NOALLOC_TABLE_128 = mf::ROPE_PMAX * (128 / 4);  // float2 entries of the d = 128 table
constexpr int NOALLOC_TABLE_64 = mf::ROPE_PMAX * (64 / 4);
static __device__ __align__(256) char scratch[NOALLOC_BYTES];
static __device__ __align__(256) float2 scratch_tables[NOALLOC_TABLE_128 + NOALLOC_TABLE_64];

// First use on a device (caller holds g_mu, the device is current): the
// arrays' device addresses, and the tables (the same host-computed values as
// mf_attn_packed's) copied in. The scratch needs no clearing: every call's
// metadata kernel rewrites the header, offsets and tile table, and the
// prologue rewrites every row of the K~ / V~ (and Q~) buffers it uses before
// the attention kernel reads them.
int noalloc_setup(DeviceState& st) {
  if (st.scratch) return MF_OK;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  void* t = nullptr;
  e = hipGetSymbolAddress(&t, HIP_SYMBOL(scratch_tables));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch_tables)");
  std::vector<float2> host = table2d_host(128, MF_ROPE_THETA);
  const std::vector<float2> t64 = table2d_host(64, MF_ROPE_THETA);
  host.insert(host.end(), t64.begin(), t64.end());
  e = hipMemcpy(t, host.data(), host.size() * sizeof(float2), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(scratch tables)");
  st.scratch_tables = static_cast<const float2*>(t);
  st.scratch = static_cast<char*>(p);
  return MF_OK;
}

}  // namespace

extern "C" {

int mf_attn_packed_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                           const int32_t* grid_hw, const int32_t* text_len, void* out, int32_t n_seg,
                           int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                           hipStream_t stream) {
  int rc = check_attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens, heads, head_dim,
                           dtype);
  if (rc) return rc;
  const mf::WsLayout l = mf::ws_layout(total_tokens, heads, head_dim, elem_bytes(dtype), n_seg, false);
  if (size_t(l.total) > NOALLOC_BYTES)
    return fail(MF_ERR_UNSUPPORTED,
                "mf_attn_packed_noalloc: these sizes need %lld bytes of scratch, the fixed maximum is %zu",
                (long long)l.total, NOALLOC_BYTES);
  int dev;
  if ((rc = current_device(&dev))) return rc;
  char* ws;
  const float2* cs;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& st = g_dev[dev];
    if ((rc = noalloc_setup(st))) return rc;
    ws = st.scratch;
    cs = st.scratch_tables + (head_dim == 128 ? 0 : NOALLOC_TABLE_128);
  }
  return run_attn(q, k, v, cu_seqlens, grid_hw, text_len, out, n_seg, total_tokens, heads, head_dim, dtype, ws, cs,
                  0, stream, nullptr, nullptr, nullptr, nullptr, false);
}

}  // extern "C"
