"""Packing metadata of a native-resolution text+image batch (oracle, fp64/int).

TEST INFRASTRUCTURE: used only by tests, the smoke check and the CPU baseline.

Source: Mage-Flow tech report, NR-MMDiT section. Images of any resolution and
aspect ratio are encoded, flattened into variable-length latent token
sequences and packed into one contiguous batch; prompt embeddings are packed
the same way instead of being padded; attention is kept inside each sample
through per-sample cumulative offsets. The editing paragraph of the same
section orders a sample's sequence as the text condition first, then the
latent tokens. The mageflow.net architecture page (section 2) encodes the
2D spatial position of every latent token.

Readings taken where the pages are silent:
* a sample is [prompt tokens ; image tokens] (text first);
* the image grid is flattened row-major (row outer, column inner);
* positions are zero-based integers with no centring or rescaling;
* prompt tokens carry position (0, 0).

Joint layout (tech report, NR-MMDiT section): text and visual tokens go
through their own modality-specific layers, and their per-token features are
concatenated sample by sample for the joint attention; both streams are packed
without padding. ``pack_joint`` builds the joint packed rows from the two
packed streams and ``unpack_joint`` splits joint rows back into them.

Editing samples (tech report, NR-MMDiT editing paragraph): the sequence is
the condition tau, then the latents of the source image(s), then the noisy
target latents, and every visual token has a 3D position (h, w, f) with f the
image index over the sources and the target. Readings: all images of a
sample share its grid (h, w) (the paragraph keeps source-target spatial
correspondence); frames are numbered 0, 1, ... in sequence order (sources
first, the target last); prompt tokens sit at (0, 0, 0).
"""
from __future__ import annotations

import numpy as np


def segment_lengths(grid_hw, text_len, frames=None) -> np.ndarray:
    """L_i = text_len_i + f_i * h_i * w_i for every sample (int64); f_i = 1
    (one image per sample) unless ``frames`` gives the images per sample."""
    g = np.asarray(grid_hw, dtype=np.int64).reshape(-1, 2)
    t = np.asarray(text_len, dtype=np.int64).reshape(-1)
    f = np.ones_like(t) if frames is None else np.asarray(frames, dtype=np.int64).reshape(-1)
    if g.shape[0] != t.shape[0] or f.shape[0] != t.shape[0]:
        raise ValueError("grid_hw, text_len and frames disagree on the number of samples")
    if (g < 1).any() or (t < 0).any() or (f < 1).any():
        raise ValueError("grid sides and frame counts must be >= 1 and prompt lengths >= 0")
    return t + f * g[:, 0] * g[:, 1]


def cu_seqlens(grid_hw, text_len, frames=None) -> np.ndarray:
    """Per-sample cumulative offsets: cu[0] = 0, cu[i+1] = cu[i] + L_i (int32)."""
    lengths = segment_lengths(grid_hw, text_len, frames)
    cu = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    for i, length in enumerate(lengths):
        cu[i + 1] = cu[i] + length
    if cu[-1] >= 2**31:
        raise ValueError("packed batch exceeds int32 token indices")
    return cu.astype(np.int32)


def token_positions(grid_hw, text_len):
    """Per-token (row, col) position and sample id of the packed sequence.

    Returns ``pos`` int32 [T, 2] and ``seg_id`` int32 [T]. Token u of sample i
    (u counted from the start of the sample) is a prompt token at (0, 0) when
    u < text_len_i; otherwise it is image token p = u - text_len_i, which sits
    at row p // w_i and column p % w_i of the latent grid.
    """
    g = np.asarray(grid_hw, dtype=np.int64).reshape(-1, 2)
    t = np.asarray(text_len, dtype=np.int64).reshape(-1)
    lengths = segment_lengths(g, t)
    total = int(lengths.sum())
    pos = np.zeros((total, 2), dtype=np.int32)
    seg = np.zeros(total, dtype=np.int32)
    start = 0
    for i in range(g.shape[0]):
        h, w, n_text = int(g[i, 0]), int(g[i, 1]), int(t[i])
        seg[start : start + n_text + h * w] = i
        # prompt tokens stay at (0, 0)
        p = np.arange(h * w, dtype=np.int64)
        pos[start + n_text : start + n_text + h * w, 0] = p // w
        pos[start + n_text : start + n_text + h * w, 1] = p % w
        start += n_text + h * w
    return pos, seg


def token_positions_3d(grid_hw, text_len, frames):
    """Per-token (row, col, frame) of a packed batch of editing samples.

    Returns ``pos3`` int32 [T, 3] and ``seg_id`` int32 [T]. Token u of sample i
    is a prompt token at (0, 0, 0) when u < text_len_i; otherwise it is visual
    token p = u - text_len_i of image f = p // (h_i w_i), at row
    (p mod h_i w_i) // w_i and column p mod w_i.
    """
    g = np.asarray(grid_hw, dtype=np.int64).reshape(-1, 2)
    t = np.asarray(text_len, dtype=np.int64).reshape(-1)
    f = np.asarray(frames, dtype=np.int64).reshape(-1)
    lengths = segment_lengths(g, t, f)
    pos = np.zeros((int(lengths.sum()), 3), dtype=np.int32)
    seg = np.zeros(int(lengths.sum()), dtype=np.int32)
    start = 0
    for i in range(g.shape[0]):
        h, w, n_text, n_img = int(g[i, 0]), int(g[i, 1]), int(t[i]), int(f[i])
        seg[start : start + int(lengths[i])] = i
        p = np.arange(n_img * h * w, dtype=np.int64)
        a = start + n_text
        pos[a : a + n_img * h * w, 0] = (p % (h * w)) // w
        pos[a : a + n_img * h * w, 1] = p % w
        pos[a : a + n_img * h * w, 2] = p // (h * w)
        start += int(lengths[i])
    return pos, seg


def pack_joint(text_stream, image_stream, grid_hw, text_len, frames=None):
    """Joint packed rows from the two packed modality streams.

    ``text_stream`` [sum T_i, ...] holds every sample's prompt rows back to back
    and ``image_stream`` [sum f_i h_i w_i, ...] every sample's image rows (grid
    row-major, images of an edit one after another). Sample i of the result is
    its T_i prompt rows, then its f_i h_i w_i image rows, at cu_seqlens[i].
    """
    lengths = segment_lengths(grid_hw, text_len, frames)
    t = np.asarray(text_len, dtype=np.int64).reshape(-1)
    text_stream = np.asarray(text_stream)
    image_stream = np.asarray(image_stream)
    if text_stream.shape[0] != t.sum() or image_stream.shape[0] != (lengths - t).sum():
        raise ValueError("stream lengths disagree with the metadata")
    if text_stream.shape[1:] != image_stream.shape[1:]:
        raise ValueError("the two streams must have the same row shape")
    out = np.empty((int(lengths.sum()),) + text_stream.shape[1:], dtype=text_stream.dtype)
    start = ts = im = 0
    for i in range(lengths.shape[0]):
        n_text, n_img = int(t[i]), int(lengths[i] - t[i])
        out[start : start + n_text] = text_stream[ts : ts + n_text]
        out[start + n_text : start + n_text + n_img] = image_stream[im : im + n_img]
        start += n_text + n_img
        ts += n_text
        im += n_img
    return out


def unpack_joint(joint, grid_hw, text_len, frames=None):
    """Inverse of ``pack_joint``: (text_stream, image_stream) from joint rows."""
    lengths = segment_lengths(grid_hw, text_len, frames)
    t = np.asarray(text_len, dtype=np.int64).reshape(-1)
    joint = np.asarray(joint)
    if joint.shape[0] != lengths.sum():
        raise ValueError("joint length disagrees with the metadata")
    text_rows, image_rows = [], []
    start = 0
    for i in range(lengths.shape[0]):
        n_text = int(t[i])
        text_rows.append(joint[start : start + n_text])
        image_rows.append(joint[start + n_text : start + int(lengths[i])])
        start += int(lengths[i])
    return np.concatenate(text_rows, axis=0), np.concatenate(image_rows, axis=0)
