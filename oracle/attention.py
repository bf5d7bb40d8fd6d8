"""Joint bidirectional attention over a packed batch (oracle, fp64).

TEST INFRASTRUCTURE: used only by tests, the smoke check and the CPU baseline.

Sources:
* mageflow.net architecture page, section 2 ("Joint Attention Mechanism") and
  section 8: text and image tokens are concatenated into one sequence and
  attend to each other in both directions (no causal mask).
* Mage-Flow tech report, NR-MMDiT section: samples are packed back to back
  and per-sample cumulative offsets keep attention inside each sample, with no
  explicit block-diagonal mask.

Readings taken where the pages are silent: multi-head attention with the same
head count for q, k and v; softmax scale 1/sqrt(head_dim); the result is the
exact softmax attention, so the oracle is that definition written out.
Large samples are processed a block of query rows at a time; every row still
sees its sample's full key set, so this is the same arithmetic per row.
"""
from __future__ import annotations

import math

import numpy as np

from . import packing, rope

ROW_BLOCK = 1024


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row-wise softmax exp(s - max) / sum, fp64; -inf entries get weight 0."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def sample_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None,
                     rows=None, row_block: int = ROW_BLOCK) -> np.ndarray:
    """softmax(Q K^T * scale) V for one sample, every head: q, k, v [L, H, d] -> [L, H, d].

    ``rows`` optionally selects query rows (indices into the sample); the result
    then has one row per selected index.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scale = default_scale(q.shape[-1]) if scale is None else scale
    if rows is not None:
        q = q[np.asarray(rows)]
    out = np.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=np.float64)
    for h in range(q.shape[1]):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for r0 in range(0, q.shape[0], row_block):
            s = (q[r0 : r0 + row_block, h, :] @ kh.T) * scale
            out[r0 : r0 + row_block, h, :] = softmax_rows(s) @ vh
    return out


def packed_attention(q, k, v, cu_seqlens, scale: float | None = None) -> np.ndarray:
    """Attention restricted to each sample of a packed batch, using the cumulative
    offsets: rows cu[i] .. cu[i+1]-1 attend only to keys cu[i] .. cu[i+1]-1."""
    q = np.asarray(q, dtype=np.float64)
    out = np.empty((q.shape[0], q.shape[1], np.shape(v)[2]), dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for i in range(cu.shape[0] - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        out[a:b] = sample_attention(q[a:b], k[a:b], v[a:b], scale)
    return out


def masked_attention(q, k, v, seg_id, scale: float | None = None) -> np.ndarray:
    """The same attention written as one dense T x T problem with a block-diagonal
    mask: a score is -inf wherever query and key belong to different samples."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scale = default_scale(q.shape[-1]) if scale is None else scale
    seg = np.asarray(seg_id)
    allowed = seg[:, None] == seg[None, :]
    out = np.empty_like(q)
    for h in range(q.shape[1]):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        s = np.where(allowed, s, -np.inf)
        out[:, h, :] = softmax_rows(s) @ v[:, h, :]
    return out


def joint_attention(q, k, v, grid_hw, text_len, theta: float = rope.DEFAULT_THETA,
                    scale: float | None = None) -> np.ndarray:
    """The whole hot path: packing metadata -> 2D RoPE on q and k -> per-sample attention."""
    cu = packing.cu_seqlens(grid_hw, text_len)
    pos, _ = packing.token_positions(grid_hw, text_len)
    if int(cu[-1]) != np.shape(q)[0]:
        raise ValueError("q has %d tokens, metadata describes %d" % (np.shape(q)[0], int(cu[-1])))
    qr = rope.rope2d(q, pos, theta)
    kr = rope.rope2d(k, pos, theta)
    return packed_attention(qr, kr, v, cu, scale)


def joint_attention_rows(q, k, v, grid_hw, text_len, tokens, theta: float = rope.DEFAULT_THETA,
                         scale: float | None = None) -> np.ndarray:
    """Output rows of ``joint_attention`` at the given packed token indices only
    (for spot checks of batches too large to evaluate whole). Returns [len(tokens), H, d]."""
    cu = packing.cu_seqlens(grid_hw, text_len)
    pos, seg = packing.token_positions(grid_hw, text_len)
    tokens = np.asarray(tokens, dtype=np.int64)
    out = np.empty((tokens.shape[0], np.shape(q)[1], np.shape(v)[2]), dtype=np.float64)
    for i in np.unique(seg[tokens]):
        a, b = int(cu[i]), int(cu[i + 1])
        sel = np.nonzero(seg[tokens] == i)[0]
        qr = rope.rope2d(np.asarray(q[a:b]), pos[a:b], theta)
        kr = rope.rope2d(np.asarray(k[a:b]), pos[a:b], theta)
        out[sel] = sample_attention(qr, kr, v[a:b], scale, rows=tokens[sel] - a)
    return out


def sample_attention_lse(q, k, scale: float | None = None) -> np.ndarray:
    """Natural-log sum-exp of each scaled score row of one sample: [L, H]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    scale = default_scale(q.shape[-1]) if scale is None else scale
    out = np.empty(q.shape[:2], dtype=np.float64)
    for h in range(q.shape[1]):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        m = np.max(s, axis=-1)
        out[:, h] = m + np.log(np.sum(np.exp(s - m[:, None]), axis=-1))
    return out


def sample_attention_backward(q, k, v, d_out, scale: float | None = None):
    """Gradients of O = softmax(Q K^T * scale) V for one sample, all heads.

    With P = softmax(S), S = Q K^T * scale and upstream gradient dO:
      dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dP * P)),
      dQ = dS K * scale,  dK = dS^T Q * scale.
    rowsum(dP * P) equals rowsum(dO * O). Returns (dq, dk, dv), each [L, H, d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    scale = default_scale(q.shape[-1]) if scale is None else scale
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for h in range(q.shape[1]):
        p = softmax_rows((q[:, h, :] @ k[:, h, :].T) * scale)
        do = d_out[:, h, :]
        dv[:, h, :] = p.T @ do
        dp = do @ v[:, h, :].T
        ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
        dq[:, h, :] = (ds @ k[:, h, :]) * scale
        dk[:, h, :] = (ds.T @ q[:, h, :]) * scale
    return dq, dk, dv


def packed_attention_backward(q, k, v, d_out, cu_seqlens, scale: float | None = None):
    """Per-sample gradients of ``packed_attention`` (samples are independent)."""
    q = np.asarray(q, dtype=np.float64)
    dq = np.empty_like(q)
    dk = np.empty(np.shape(k), dtype=np.float64)
    dv = np.empty(np.shape(v), dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for i in range(cu.shape[0] - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        dq[a:b], dk[a:b], dv[a:b] = sample_attention_backward(q[a:b], k[a:b], v[a:b], d_out[a:b], scale)
    return dq, dk, dv


def joint_attention_lse(q, k, grid_hw, text_len, theta: float = rope.DEFAULT_THETA,
                        scale: float | None = None) -> np.ndarray:
    """Row log-sum-exp of the joint path's scaled scores, [H, T] (natural log):
    2D RoPE on q and k, then ``sample_attention_lse`` per sample."""
    cu = packing.cu_seqlens(grid_hw, text_len)
    pos, _ = packing.token_positions(grid_hw, text_len)
    qr = rope.rope2d(q, pos, theta)
    kr = rope.rope2d(k, pos, theta)
    out = np.empty((np.shape(q)[1], np.shape(q)[0]), dtype=np.float64)
    for i in range(cu.shape[0] - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        out[:, a:b] = sample_attention_lse(qr[a:b], kr[a:b], scale).T
    return out


def joint_attention_backward(q, k, v, d_out, grid_hw, text_len, theta: float = rope.DEFAULT_THETA,
                             scale: float | None = None):
    """Gradients of ``joint_attention`` with respect to the unrotated q, k and v.
    The rotation is linear and orthogonal, so the gradient of the rotated input is
    mapped back by the inverse rotation."""
    cu = packing.cu_seqlens(grid_hw, text_len)
    pos, _ = packing.token_positions(grid_hw, text_len)
    qr = rope.rope2d(q, pos, theta)
    kr = rope.rope2d(k, pos, theta)
    dqr, dkr, dv = packed_attention_backward(qr, kr, v, d_out, cu, scale)
    return rope.rope2d_inverse(dqr, pos, theta), rope.rope2d_inverse(dkr, pos, theta), dv


# ---------------------------------------------------------------- editing (frame-aware) variant
#
# Tech report, NR-MMDiT editing paragraph: an editing sample is the condition
# followed by the source latents and the target latents, and the 2D RoPE is
# extended with the image index f: every visual token sits at (h, w, f).
# ``split`` gives the channels turned by row, column and frame (contiguous
# blocks in that order; the pages do not fix it).


def _positions_3d(grid_hw, text_len, frames):
    cu = packing.cu_seqlens(grid_hw, text_len, frames)
    pos3, _ = packing.token_positions_3d(grid_hw, text_len, frames)
    return cu, pos3


def joint_attention_3d(q, k, v, grid_hw, text_len, frames, split, theta: float = rope.DEFAULT_THETA,
                       scale: float | None = None) -> np.ndarray:
    """Packed joint attention of editing samples with frame-aware RoPE."""
    cu, pos3 = _positions_3d(grid_hw, text_len, frames)
    if int(cu[-1]) != np.shape(q)[0]:
        raise ValueError("q has %d tokens, metadata describes %d" % (np.shape(q)[0], int(cu[-1])))
    return packed_attention(rope.rope3d(q, pos3, split, theta), rope.rope3d(k, pos3, split, theta), v, cu, scale)


def joint_attention_3d_lse(q, k, grid_hw, text_len, frames, split, theta: float = rope.DEFAULT_THETA,
                           scale: float | None = None) -> np.ndarray:
    """Row log-sum-exp [H, T] of ``joint_attention_3d``'s scaled scores."""
    cu, pos3 = _positions_3d(grid_hw, text_len, frames)
    qr, kr = rope.rope3d(q, pos3, split, theta), rope.rope3d(k, pos3, split, theta)
    out = np.empty((np.shape(q)[1], np.shape(q)[0]), dtype=np.float64)
    for i in range(cu.shape[0] - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        out[:, a:b] = sample_attention_lse(qr[a:b], kr[a:b], scale).T
    return out


def joint_attention_3d_backward(q, k, v, d_out, grid_hw, text_len, frames, split,
                                theta: float = rope.DEFAULT_THETA, scale: float | None = None):
    """Gradients of ``joint_attention_3d`` with respect to the unrotated q, k and v."""
    cu, pos3 = _positions_3d(grid_hw, text_len, frames)
    qr, kr = rope.rope3d(q, pos3, split, theta), rope.rope3d(k, pos3, split, theta)
    dqr, dkr, dv = packed_attention_backward(qr, kr, v, d_out, cu, scale)
    return rope.rope3d_inverse(dqr, pos3, split, theta), rope.rope3d_inverse(dkr, pos3, split, theta), dv
