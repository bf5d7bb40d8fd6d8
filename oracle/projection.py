"""Modality-specific RMSNorm + packed QKV projection of a packed batch (oracle, fp64).

TEST INFRASTRUCTURE: used only by tests, the smoke check and the CPU baseline.

Sources: Mage-Flow tech report, NR-MMDiT section (each MMDiT block keeps
separate normalization and projection layers for the text stream and the
visual stream; the two are concatenated only for the joint attention);
mageflow.net architecture page, section 7 (the RMSNorm layers are fused and
the linear projections packed).

Readings taken where the pages are silent:
* the normalization is RMSNorm over the hidden channels,
  h = x / sqrt(mean(x^2) + eps) * gamma, with a gain per modality and
  eps = 1e-6, and no adaptive (timestep) modulation;
* "packed" projection: one weight per modality producing q, k and v together,
  stored like a linear layer's weight, [3 * heads * head_dim][hidden], rows
  [0, HD) give q, [HD, 2HD) k and [2HD, 3HD) v; no bias;
* a token is "text" when it is one of its sample's prompt tokens, "visual"
  otherwise (all images of an editing sample included).
"""
from __future__ import annotations

import numpy as np

from .packing import segment_lengths


def rmsnorm(x, gamma, eps: float = 1e-6):
    """x / sqrt(mean(x^2, last axis) + eps) * gamma."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(gamma, dtype=np.float64)


def text_mask(grid_hw, text_len, frames=None):
    """Boolean [T]: True for prompt tokens of the packed batch."""
    lengths = segment_lengths(grid_hw, text_len, frames)
    t = np.asarray(text_len, dtype=np.int64).reshape(-1)
    mask = np.zeros(int(lengths.sum()), dtype=bool)
    start = 0
    for L, n_text in zip(lengths, t):
        mask[start:start + int(n_text)] = True
        start += int(L)
    return mask


def rmsnorm_qkv(x, w_txt, w_img, gamma_txt, gamma_img, grid_hw, text_len, heads: int, head_dim: int,
                frames=None, eps: float = 1e-6):
    """q, k, v [T, heads, head_dim] of the packed hidden states x [T, hidden]:
    every token is normalized with its modality's gain and projected with its
    modality's packed weight."""
    x = np.asarray(x, dtype=np.float64)
    mask = text_mask(grid_hw, text_len, frames)
    if mask.shape[0] != x.shape[0]:
        raise ValueError("x has %d tokens, metadata describes %d" % (x.shape[0], mask.shape[0]))
    y = np.empty((x.shape[0], 3 * heads * head_dim), dtype=np.float64)
    for m, w, g in ((mask, w_txt, gamma_txt), (~mask, w_img, gamma_img)):
        if m.any():
            y[m] = rmsnorm(x[m], g, eps) @ np.asarray(w, dtype=np.float64).T
    hd = heads * head_dim
    return tuple(y[:, i * hd:(i + 1) * hd].reshape(-1, heads, head_dim) for i in range(3))
