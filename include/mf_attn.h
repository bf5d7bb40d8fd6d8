/*
 * mf_attn.h -- packed joint text+image attention with 2D RoPE (gfx950 / MI355X).
 *
 * C ABI of libmfattn.so. Every pointer argument named "device" is HIP device
 * memory owned by the caller; the library never frees caller memory. All
 * work is enqueued on the caller's stream and returns without waiting, except
 * where a function says it synchronizes. Functions return an mf_status; on a
 * negative status nothing was enqueued and mf_last_error() holds a message.
 *
 * HIP graph capture: the first call of an entry point on a device may
 * allocate (library workspace, status word) and upload the RoPE tables with
 * synchronous copies. After one eager call with the same or larger sizes, the
 * enqueuing calls launch kernels only (no host synchronization, allocation or
 * memset) and can be captured into a graph and replayed. A later call that
 * needs a larger library workspace reallocates it, which invalidates graphs
 * that captured the old one; mf_attn_packed_ws with a caller-owned workspace
 * avoids that.
 *
 * Operation (sources, by page and section):
 *  - Mage-Flow tech report, NR-MMDiT section: text and image tokens of one
 *    sample are concatenated and processed by joint self-attention; samples
 *    of different resolutions and prompt lengths are packed back to back with
 *    no padding, and per-sample cumulative offsets keep attention inside each
 *    sample without an explicit block-diagonal mask. The editing paragraph of
 *    that section puts the text condition before the latent tokens.
 *  - mageflow.net architecture page, section 2: joint bidirectional attention
 *    and 2D rotary position embeddings; section 8: text tokens are updated by
 *    image tokens too (no causal mask).
 *  - Mage-Flow tech report, Mage-VAE section: 16x spatial reduction, so an
 *    image of H x W pixels has an (H/16) x (W/16) latent grid.
 *
 * Conventions fixed by this library where the pages are silent:
 *  - sample i = [text_len[i] prompt tokens ; h_i * w_i image tokens], the grid
 *    flattened row-major; L_i = text_len[i] + h_i * w_i;
 *    cu_seqlens[0] = 0, cu_seqlens[i+1] = cu_seqlens[i] + L_i; T = cu_seqlens[n];
 *  - prompt tokens sit at position (0, 0); image token p at (p / w, p % w);
 *  - 2D RoPE: channels [0, d/2) turn with the row, [d/2, d) with the column;
 *    adjacent pairs (2j, 2j+1) inside each half, frequency theta^(-2j/(d/2));
 *    pair (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos); queries and keys
 *    only; theta = 10000 in mf_attn_packed;
 *  - softmax scale 1/sqrt(d); equal head counts for q, k, v.
 *
 * Tensor layout: q, k, v and out are contiguous [T][heads][head_dim] with
 * elements of the given dtype (MF_BF16: bfloat16 bit patterns; MF_F32:
 * float), except in mf_attn_packed_strided, which takes strided descriptors.
 * Metadata arrays are contiguous int32 in device memory.
 * Supported: head_dim in {64, 128}; 1 <= heads <= 256; 1 <= n_seg <= 4096;
 * 1 <= h, w <= 512; 0 <= text_len; T < 2^31 (and every buffer < 2^31 elements
 * per head).
 */
#ifndef MF_ATTN_H
#define MF_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MF_OK = 0,
  MF_ERR_INVALID_ARG = -1, /* bad scalar, null or overlapping pointer */
  MF_ERR_METADATA = -2,    /* cu_seqlens / grid / prompt lengths inconsistent (device-detected) */
  MF_ERR_UNSUPPORTED = -3, /* head_dim, dtype or size outside the supported set */
  MF_ERR_HIP = -4,         /* a HIP runtime call failed */
  MF_ERR_OOM = -5          /* workspace allocation failed */
} mf_status;

typedef enum { MF_BF16 = 0, MF_F32 = 1 } mf_dtype;

#define MF_MAX_SEGMENTS 4096
#define MF_MAX_GRID_SIDE 512
#define MF_ROPE_THETA 10000.0f

/*
 * Strided tensor descriptor (host struct, owned by the caller, read during
 * the call only). Element (token t, head h, channel c) of the tensor is at
 * data + (t * stride_token + h * stride_head + c) elements; channels are
 * contiguous. dtype is MF_BF16 or MF_F32.
 */
typedef struct {
  void* data;
  int32_t dtype;
  int32_t tokens;
  int32_t heads;
  int32_t head_dim;
  int64_t stride_token;
  int64_t stride_head;
} mf_tensor;

/* Library version as major*10000 + minor*100 + patch. */
int mf_version(void);

/* Message of the last failing call on this host thread ("" if none). */
const char* mf_last_error(void);

/*
 * Packed joint attention with 2D RoPE: out = per-sample softmax(R(q) R(k)^T /
 * sqrt(d)) v, where R is the 2D rotation at each token's (row, col).
 *   q, k, v   device [total_tokens][heads][head_dim], dtype
 *   cu_seqlens device int32 [n_seg + 1], must equal the prefix sums of L_i
 *   grid_hw   device int32 [n_seg][2] = (h, w) latent grid of each image
 *   text_len  device int32 [n_seg]
 *   out       device [total_tokens][heads][head_dim], dtype; must not overlap
 *             q, k, v or the metadata
 * The library checks the metadata on the device (L_i >= 1, sides in range,
 * cu_seqlens consistent, cu_seqlens[n_seg] == total_tokens). On a mismatch no
 * output is written and mf_get_device_error() reports MF_ERR_METADATA.
 * Uses a library-owned workspace per device (grown on demand, never shrunk,
 * freed at process exit). Calls on that workspace are ordered on the device:
 * a call enqueued on a stream other than the previous call's first makes its
 * stream wait for that call (an event; the host is not blocked), so calls on
 * several streams of one device run one after the other. Calls enqueued while
 * their stream is being captured into a graph are not ordered this way, and
 * replays of such a graph must not overlap other calls on the device. Calls
 * that should run concurrently use mf_attn_packed_ws with separate
 * workspaces.
 * Results are deterministic (no atomics). For bf16, when the last round of
 * (256-query tile, head) units would fill the device poorly and its units are
 * long, those units are split over key ranges and a second kernel merges the
 * pieces in a fixed order; this happens only for batches whose mean sample
 * length is at least 8129 tokens, and it changes the rounding of the split
 * units (not the result beyond it). MF_ATTN_SPLIT=0 in the environment (read
 * at the first call on a device) turns the split off.
 */
int mf_attn_packed(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                   const int32_t* grid_hw, const int32_t* text_len, void* out, int32_t n_seg,
                   int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                   hipStream_t stream);

/*
 * mf_attn_packed that also records four caller-created hipEvent_t on `stream`
 * (events[0..3]): before the metadata kernel, after it, after the RoPE
 * prologue and after the attention kernel, so each stage can be timed with
 * hipEventElapsedTime. Otherwise identical to mf_attn_packed.
 */
int mf_attn_packed_profiled(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                            const int32_t* grid_hw, const int32_t* text_len, void* out,
                            int32_t n_seg, int64_t total_tokens, int32_t heads, int32_t head_dim,
                            int32_t dtype, hipEvent_t const* events, hipStream_t stream);

/* Bytes of workspace mf_attn_packed_ws needs for these sizes (0 if unsupported). */
size_t mf_workspace_bytes(int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                          int32_t n_seg);

/*
 * Same as mf_attn_packed with a caller-provided device workspace of at least
 * mf_workspace_bytes(...) bytes, 256-byte aligned. The workspace must stay
 * alive until the enqueued work finishes; nothing is allocated.
 */
int mf_attn_packed_ws(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                      const int32_t* grid_hw, const int32_t* text_len, void* out, int32_t n_seg,
                      int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mf_attn_packed on strided tensors, e.g. views of one fused [T][3][heads][d]
 * projection output (stride_token 3 * heads * d) or of a head-major
 * [heads][T][d] buffer, without a copy. Same operation, metadata checks,
 * workspace and results as mf_attn_packed (bit for bit on the same values).
 *   q, k, v, out  descriptors with equal dtype, tokens, heads and head_dim;
 *                 data 16-byte aligned; both strides at least head_dim and
 *                 multiples of 16 bytes; q, k and v may overlap each other
 *   out           must be one-to-one (stride_head >= head_dim and
 *                 stride_token >= (heads - 1) * stride_head + head_dim, or
 *                 the head-major analogue), and its span must not overlap
 *                 the spans of q, k, v or the metadata
 * The forward only: mf_attn_packed_lse, the backward and the frame-aware
 * variants take contiguous tensors.
 */
int mf_attn_packed_strided(const mf_tensor* q, const mf_tensor* k, const mf_tensor* v, const int32_t* cu_seqlens,
                           const int32_t* grid_hw, const int32_t* text_len, int32_t n_seg, const mf_tensor* out,
                           hipStream_t stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, checks and results as mf_attn_packed, but the
 * workspace is a fixed static device array of MF_NOALLOC_SCRATCH_BYTES bytes
 * (each device the library runs on holds its own copy from the first call on
 * it until the process ends), so no call allocates or frees anything.
 *  - Limit: header and metadata plus the rotated-key and transposed-value
 *    buffers (MF_F32: also the rotated queries) of heads x rows x head_dim
 *    elements each must fit, rows = the sum over samples of L_i rounded up to
 *    64, plus 192. bf16 with 24 heads x 128: about 21,600 packed tokens (the
 *    1024x1024, 2048x2048 and mixed-aspect batches fit). Larger batches return
 *    MF_ERR_UNSUPPORTED with the bytes they would need.
 *  - Never splits a poorly filled last round (the split needs partial-result
 *    slots), so results equal mf_attn_packed's bit for bit wherever that call
 *    does not split either (mean sample length below 8129 tokens), and are
 *    within rounding of them elsewhere.
 *  - The first call on a device does a one-time synchronous setup: it looks
 *    up the static arrays' device addresses and copies the RoPE cos/sin tables
 *    into one of them (no allocation). Make one call before capturing.
 *  - Every call on a device uses that device's one scratch array and leaves
 *    its contents behind. Calls that overlap on one device (two streams,
 *    concurrent graph replays) race on it and give wrong results; order them
 *    on one stream.
 * A metadata mismatch behaves as for mf_attn_packed (nothing written,
 * reported by mf_get_device_error).
 */
#define MF_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int mf_attn_packed_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                           const int32_t* grid_hw, const int32_t* text_len, void* out, int32_t n_seg,
                           int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                           hipStream_t stream);

/*
 * Forward for training: mf_attn_packed that also stores each query row's
 * log-sum-exp of its scaled scores, the statistic the backward recomputes P
 * from (no score matrix is kept).
 *   lse  device float [heads][total_tokens]: ln sum_k exp(q~.k~ / sqrt(d)) over
 *        the row's own sample; must not overlap the other arguments
 * Same sources, checks and workspace as mf_attn_packed.
 */
int mf_attn_packed_lse(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                       const int32_t* grid_hw, const int32_t* text_len, void* out, float* lse,
                       int32_t n_seg, int64_t total_tokens, int32_t heads, int32_t head_dim,
                       int32_t dtype, hipStream_t stream);

/*
 * Packed backward: gradients of mf_attn_packed with respect to q, k and v.
 * Sources: Mage-Flow tech report, NR-MMDiT section (training on packed
 * native-resolution batches, attention restricted to each sample by its
 * cumulative offsets); mageflow.net architecture page, section 2 (2D RoPE).
 * With P the per-sample softmax, D = rowsum(d_out * out):
 *   dv = P^T d_out, dX = P * (d_out v^T - D), dq = R^T (dX R(k)) / sqrt(d),
 *   dk = R^T (dX^T R(q)) / sqrt(d).
 *   q, k, v, out, d_out  device [total_tokens][heads][head_dim], MF_BF16
 *               (out is the forward's output; d_out the upstream gradient)
 *   lse         device float [heads][total_tokens] from mf_attn_packed_lse
 *   cu_seqlens, grid_hw, text_len  as for mf_attn_packed
 *   dq, dk, dv  device [total_tokens][heads][head_dim], MF_BF16, written in
 *               full; must not overlap each other, the inputs or the metadata
 * bf16 only (MF_F32 returns MF_ERR_UNSUPPORTED); head_dim 64 or 128. The
 * metadata is checked on the device as for the forward: on a mismatch nothing
 * is written and mf_get_device_error() reports MF_ERR_METADATA. Uses a second
 * library-owned per-device workspace (mf_bwd_workspace_bytes), with the same
 * stream-order rule as mf_attn_packed. Deterministic: no atomics. When the
 * last round of (128-key block, head) units of the dK/dV kernel would fill the
 * device poorly and its units are long, those units are split over query
 * ranges and the pieces' fp32 partial sums are added in a fixed order; this
 * happens only for batches whose mean sample length is at least 1985 tokens
 * and changes the rounding of dk and dv in the split units. The dQ kernel's
 * (256-query tile, head) units split the same way over key ranges, for
 * batches whose mean sample length is at least 8129 tokens (rounding of dq in
 * the split units). MF_ATTN_SPLIT=0 turns both off, like the forward's split.
 */
int mf_attn_packed_bwd(const void* q, const void* k, const void* v, const void* out, const void* d_out,
                       const float* lse, const int32_t* cu_seqlens, const int32_t* grid_hw,
                       const int32_t* text_len, void* dq, void* dk, void* dv, int32_t n_seg,
                       int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                       hipStream_t stream);

/*
 * mf_attn_packed_bwd that records four caller-created hipEvent_t on `stream`:
 * before the metadata kernel, after the backward prologue, after the dK/dV
 * kernel and after the dQ kernel. Otherwise identical.
 */
int mf_attn_packed_bwd_profiled(const void* q, const void* k, const void* v, const void* out,
                                const void* d_out, const float* lse, const int32_t* cu_seqlens,
                                const int32_t* grid_hw, const int32_t* text_len, void* dq, void* dk,
                                void* dv, int32_t n_seg, int64_t total_tokens, int32_t heads,
                                int32_t head_dim, int32_t dtype, hipEvent_t const* events,
                                hipStream_t stream);

/* Bytes of the backward's library-owned workspace for these sizes (0 if unsupported). */
size_t mf_bwd_workspace_bytes(int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t n_seg);

/*
 * Frame-aware variants for editing samples. Source: Mage-Flow tech report,
 * NR-MMDiT section, editing paragraph: the sequence of an editing sample is
 * the condition, then the source image latents, then the target latents, and
 * the 2D RoPE gains the image index f, so every visual token sits at
 * (h, w, f). Readings (the pages fix neither): all images of a sample share
 * its grid; frames are numbered 0, 1, ... in sequence order; prompt tokens
 * sit at (0, 0, 0); the head dimension is split into three contiguous channel
 * blocks turned by row, column and frame, each with its own frequency ladder
 * theta^(-2j/m) (m = channels of the block), adjacent pairs as in 2D.
 *   frames      device int32 [n_seg]: images per sample, 1 .. 512
 *               (L_i = text_len_i + frames_i * h_i * w_i)
 *   split_row, split_col, split_frame  host: channels per block, even, >= 0,
 *               summing to head_dim; (head_dim/2, head_dim/2, 0) with all
 *               frames 1 gives exactly mf_attn_packed's result
 *   lse         optional (NULL allowed) device float [heads][total_tokens]
 * Everything else as mf_attn_packed / mf_attn_packed_lse.
 */
int mf_attn_packed_3d(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                      const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames, int32_t split_row,
                      int32_t split_col, int32_t split_frame, void* out, float* lse, int32_t n_seg,
                      int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype, hipStream_t stream);

/* Backward of mf_attn_packed_3d (lse required), as mf_attn_packed_bwd. */
int mf_attn_packed_3d_bwd(const void* q, const void* k, const void* v, const void* out, const void* d_out,
                          const float* lse, const int32_t* cu_seqlens, const int32_t* grid_hw,
                          const int32_t* text_len, const int32_t* frames, int32_t split_row, int32_t split_col,
                          int32_t split_frame, void* dq, void* dk, void* dv, int32_t n_seg, int64_t total_tokens,
                          int32_t heads, int32_t head_dim, int32_t dtype, hipStream_t stream);

/*
 * Metadata of editing samples: as mf_build_metadata with frames, and pos_out
 * device int32 [total_tokens][3] = (row, col, frame).
 */
int mf_build_metadata_3d(int32_t n_seg, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                         int32_t* cu_seqlens_out, int32_t* pos_out, int32_t* seg_id_out, int64_t total_tokens,
                         hipStream_t stream);

/*
 * Frame-aware RoPE alone: x_out = R(pos) x_in with pos device int32
 * [total_tokens][3] = (row, col, frame), each in [0, 512), and the channel
 * split above. Otherwise as mf_rope_2d.
 */
int mf_rope_3d(const void* x_in, void* x_out, const int32_t* pos, int64_t total_tokens, int32_t heads,
               int32_t head_dim, int32_t dtype, float theta, int32_t split_row, int32_t split_col,
               int32_t split_frame, hipStream_t stream);

/*
 * Packing metadata alone (same conventions as above).
 *   grid_hw, text_len  device int32 inputs
 *   cu_seqlens_out     device int32 [n_seg + 1]
 *   pos_out            device int32 [total_tokens][2] = (row, col)
 *   seg_id_out         device int32 [total_tokens]
 * total_tokens is the capacity of pos_out / seg_id_out and must equal the
 * packed length; otherwise nothing past the capacity is written and the
 * device error flag reports MF_ERR_METADATA.
 */
int mf_build_metadata(int32_t n_seg, const int32_t* grid_hw, const int32_t* text_len,
                      int32_t* cu_seqlens_out, int32_t* pos_out, int32_t* seg_id_out,
                      int64_t total_tokens, hipStream_t stream);

/*
 * Joint-layout pack and unpack. Source: Mage-Flow tech report, NR-MMDiT
 * section: text and visual tokens pass through modality-specific layers and
 * are concatenated, sample by sample, for the joint attention; prompts and
 * images are each packed without padding. The text stream holds every
 * sample's prompt rows back to back (text_tokens = sum of text_len rows), the
 * image stream every sample's image rows (grid row-major; the frames images
 * of an edit one after another; total_tokens - text_tokens rows), and the
 * joint tensor sample i's prompt rows then its image rows at cu_seqlens[i]:
 *   joint[cu[i] + u] = u < T_i ? text[tcu[i] + u] : image[cu[i] - tcu[i] + u - T_i],
 * tcu[i] = T_0 + ... + T_{i-1}. mf_unpack_joint is the inverse map (e.g. the
 * attention output back to the two streams). Pure copies, bit-exact.
 *   n_tensors   1 .. 4 tensors moved by one launch (e.g. q, k, v)
 *   text, image, joint  host arrays of n_tensors device pointers; each tensor
 *               [rows][heads][head_dim] contiguous, dtype, 16-byte aligned; a
 *               stream with no rows may be NULL
 *   cu_seqlens, grid_hw, text_len  device int32 as for mf_attn_packed;
 *               frames device int32 [n_seg] or NULL (one image per sample)
 * The outputs must not overlap each other, the inputs or the metadata. The
 * metadata is checked on the device (cu_seqlens against the prefix sums of
 * text_len + frames * h * w, sides in range, cu_seqlens[n_seg] ==
 * total_tokens, the prompts adding up to text_tokens); on a mismatch nothing
 * is written and mf_get_device_error() reports MF_ERR_METADATA. One kernel
 * launch, no library workspace (only the device's status word).
 */
int mf_pack_joint(int32_t n_tensors, const void* const* text, const void* const* image, void* const* joint,
                  const int32_t* cu_seqlens, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                  int32_t n_seg, int64_t total_tokens, int64_t text_tokens, int32_t heads, int32_t head_dim,
                  int32_t dtype, hipStream_t stream);
int mf_unpack_joint(int32_t n_tensors, const void* const* joint, void* const* text, void* const* image,
                    const int32_t* cu_seqlens, const int32_t* grid_hw, const int32_t* text_len, const int32_t* frames,
                    int32_t n_seg, int64_t total_tokens, int64_t text_tokens, int32_t heads, int32_t head_dim,
                    int32_t dtype, hipStream_t stream);

/*
 * 2D RoPE alone: x_out = R(pos) x_in, per token and head.
 *   x_in, x_out device [total_tokens][heads][head_dim], dtype (may be the same buffer)
 *   pos         device int32 [total_tokens][2], each in [0, 512)
 * fp32 arithmetic with a cos/sin table computed on the host in double
 * precision; bf16 results are rounded to nearest even. Positions outside
 * [0, 512) leave the row unchanged and set the device error flag.
 */
int mf_rope_2d(const void* x_in, void* x_out, const int32_t* pos, int64_t total_tokens,
               int32_t heads, int32_t head_dim, int32_t dtype, float theta, hipStream_t stream);

/*
 * Modality-specific RMSNorm + packed QKV projection, the prologue that feeds
 * the joint attention. Sources: Mage-Flow tech report, NR-MMDiT section
 * (separate normalization and projection layers for the text and the visual
 * stream of every MMDiT block); mageflow.net architecture page, section 7
 * (fused RMSNorm, packed linear projections). Readings: RMSNorm over the
 * hidden channels with a gain per modality, no modulation, no bias; prompt
 * tokens are "text", every other token "visual".
 *
 * mf_qkv_fold_weights folds the gains into the weights once per weight update:
 *   w_txt, w_img    device bf16 [3 * heads * head_dim][hidden], a linear
 *                   layer's weight (rows: q, then k, then v, head-major)
 *   gamma_txt, gamma_img  device float [hidden]
 *   w_out           device bf16, 2 * 3 * heads * head_dim * hidden elements
 *                   holding W'_m[n][c] = bf16(gamma_m[c] * w_m[n][c]) (m = 0
 *                   text, 1 visual) in the projection's tiled order: stacked
 *                   row R = m * 3HD + n, 8-channel chunk g = c / 8, stored as
 *                   16-byte chunk ((R / 256) * (hidden / 64) + g / 8) * 2048
 *                   + (g % 8) * 256 + R % 256
 * hidden a multiple of 64; heads * head_dim a multiple of 256.
 */
int mf_qkv_fold_weights(const void* w_txt, const void* w_img, const float* gamma_txt, const float* gamma_img,
                        int32_t hidden, int32_t heads, int32_t head_dim, void* w_out, hipStream_t stream);

/*
 * mf_qkv_rmsnorm: for every token t of modality m,
 *   [q | k | v][t] = (x[t] / sqrt(mean(x[t]^2) + eps)) (w_folded[m])^T
 * (fp32 statistics and accumulation, bf16 results).
 *   x           device bf16 [total_tokens][hidden], packed like the attention input
 *   w_folded    device bf16 from mf_qkv_fold_weights
 *   cu_seqlens, grid_hw, text_len  as for mf_attn_packed; frames (device int32
 *               [n_seg], NULL = one image per sample) as for mf_attn_packed_3d
 *   q, k, v     device bf16 [total_tokens][heads][head_dim], the attention's inputs
 * The metadata is checked on the device; on a mismatch nothing is written and
 * mf_get_device_error() reports MF_ERR_METADATA. Uses a library-owned
 * per-device workspace (row lists, 1/rms and a tiled copy of x, about
 * 12 + 2 * hidden bytes per token), same stream-order rule as mf_attn_packed.
 * Deterministic (no atomics); the work schedule (a poorly filled last round
 * of GEMM tiles runs as half tiles, off with MF_ATTN_SPLIT=0) never changes
 * the summation order, so results do not depend on it.
 */
int mf_qkv_rmsnorm(const void* x, const void* w_folded, const int32_t* cu_seqlens, const int32_t* grid_hw,
                   const int32_t* text_len, const int32_t* frames, int32_t n_seg, int64_t total_tokens, int32_t hidden,
                   int32_t heads, int32_t head_dim, float eps, void* q, void* k, void* v, hipStream_t stream);

/* mf_qkv_rmsnorm recording three hipEvent_t: before, after the statistics, after the projection. */
int mf_qkv_rmsnorm_profiled(const void* x, const void* w_folded, const int32_t* cu_seqlens, const int32_t* grid_hw,
                            const int32_t* text_len, const int32_t* frames, int32_t n_seg, int64_t total_tokens,
                            int32_t hidden, int32_t heads, int32_t head_dim, float eps, void* q, void* k, void* v,
                            hipEvent_t const* events, hipStream_t stream);

/*
 * Guided rectified-flow Euler step over a packed classifier-free-guidance batch.
 * Sources: Mage-Flow tech report, NR-MMDiT section (the conditional and the
 * unconditional branch are packed together and evaluated in one forward pass);
 * mageflow.net architecture page, section 3 (straight rectified-flow paths
 * sampled with Euler steps). The guided velocity is v_u + s * (v_c - v_u) (the
 * pages do not print it; this is the standard form), and the step is
 *   z <- z + dt * (v_u + guidance * (v_c - v_u)).
 *   z           device float [image_tokens][channels]: the images' latent tokens
 *               back to back in image order, each image's grid row-major;
 *               updated in place
 *   v           device [total_tokens][channels], dtype: the velocity predicted
 *               for every token of the packed batch
 *   cu_seqlens, grid_hw, text_len  device int32, the packed batch's metadata
 *               (same conventions as mf_attn_packed, n_seg samples)
 *   cond_seg    device int32 [n_img]: sample holding image b with its prompt
 *   uncond_seg  device int32 [n_img]: sample holding image b without it, or -1
 *               for no guidance (then the step uses v_c alone)
 * Image b owns h*w tokens of z, (h, w) = grid_hw[cond_seg[b]]. channels is a
 * positive multiple of 8 (at most 4096), image_tokens * channels / 8 < 2^31, z
 * and v are 16-byte aligned, n_img <= MF_MAX_SEGMENTS and grid sides are at
 * most MF_MAX_GRID_SIDE. One kernel launch; it first checks on the device that
 * every index is in range, that both samples of an image have the same grid,
 * that cu_seqlens agrees with grid_hw/text_len for the samples used and ends
 * inside total_tokens, and that the images' tokens add up to image_tokens. If
 * any check fails nothing is written and the device flag read by
 * mf_get_device_error is set. Arithmetic in fp32. Uses no library workspace,
 * so calls on different streams that touch disjoint z buffers may overlap.
 */
int mf_rf_cfg_euler_step(float* z, const void* v, const int32_t* cu_seqlens, const int32_t* grid_hw,
                         const int32_t* text_len, int32_t n_seg, int64_t total_tokens,
                         const int32_t* cond_seg, const int32_t* uncond_seg, int32_t n_img,
                         int64_t image_tokens, int32_t channels, int32_t dtype, float guidance,
                         float dt, hipStream_t stream);

/*
 * Synchronizes `stream`, then returns MF_ERR_METADATA if the last enqueued
 * metadata check on any of this device's library workspaces (forward,
 * backward, projection, the allocation-free forward's scratch) or the sticky
 * flag of the standalone metadata, RoPE and sampler calls failed, else MF_OK.
 * Each failure is reported once: the sticky flag is cleared and a failed
 * workspace check is marked as reported (the next call on that workspace
 * checks afresh), so a later call that fails nothing returns MF_OK.
 */
int mf_get_device_error(hipStream_t stream);

/* Same, for a caller-provided workspace of mf_attn_packed_ws. */
int mf_get_workspace_error(const void* workspace, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MF_ATTN_H */
