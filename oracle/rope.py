"""2D rotary position embedding (oracle, fp64).

TEST INFRASTRUCTURE: used only by tests, the smoke check and the CPU baseline.

Source: mageflow.net architecture page, section 2 ("Rotary Position
Embeddings (2D RoPE)"): 2D spatial positions are encoded natively, for any
aspect ratio, with no interpolation onto a fixed grid. The Mage-Flow tech
report (editing paragraph of the NR-MMDiT section) extends the same 2D RoPE
with a frame index f, giving (h, w, f) positions; ``rope3d`` below is that
extension.

The pages do not fix the layout. Reading taken (the standard rotary form,
one rotation per pair of channels):
* the head dimension d is split in two halves; the first half [0, d/2) is
  rotated by the row index, the second half [d/2, d) by the column index;
* inside a half of size d/2, channel pairs are adjacent: (2j, 2j+1) for
  j = 0 .. d/4 - 1, with angular frequency w_j = theta ** (-2j / (d/2));
* pair (x0, x1) at angle phi becomes (x0 cos phi - x1 sin phi,
  x0 sin phi + x1 cos phi);
* theta = 10000; rotation applies to queries and keys, never to values.
"""
from __future__ import annotations

import numpy as np

DEFAULT_THETA = 10000.0


def axis_frequencies(dims_per_axis: int, theta: float = DEFAULT_THETA) -> np.ndarray:
    """w_j = theta ** (-2j / m) for j = 0 .. m/2 - 1, m = channels given to one axis."""
    if dims_per_axis % 2:
        raise ValueError("channels per axis must be even")
    j = np.arange(dims_per_axis // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / dims_per_axis)


def _rotate_pairs(x: np.ndarray, angle: np.ndarray) -> np.ndarray:
    """Rotate adjacent channel pairs of x [T, H, 2P] by angle [T, P] (same angle for every head)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.cos(angle)[:, None, :]
    s = np.sin(angle)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def angles_2d(pos: np.ndarray, head_dim: int, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Rotation angle of every channel pair: [T, d/2]. Pairs 0 .. d/4-1 use the row,
    pairs d/4 .. d/2-1 use the column, both with the frequencies of a d/2-channel axis."""
    if head_dim % 4:
        raise ValueError("head_dim must be a multiple of 4 for 2D RoPE")
    pos = np.asarray(pos, dtype=np.float64).reshape(-1, 2)
    freqs = axis_frequencies(head_dim // 2, theta)
    row = pos[:, 0:1] * freqs[None, :]
    col = pos[:, 1:2] * freqs[None, :]
    return np.concatenate([row, col], axis=1)


def rope2d(x: np.ndarray, pos: np.ndarray, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Apply 2D RoPE to x [T, H, d] at integer positions pos [T, 2] = (row, col)."""
    x = np.asarray(x, dtype=np.float64)
    return _rotate_pairs(x, angles_2d(pos, x.shape[-1], theta))


def rope2d_inverse(x: np.ndarray, pos: np.ndarray, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Transpose (= inverse) of ``rope2d``: rotation by the negated angles. Used to map
    gradients taken in the rotated space back to the unrotated inputs."""
    x = np.asarray(x, dtype=np.float64)
    return _rotate_pairs(x, -angles_2d(pos, x.shape[-1], theta))


def angles_3d(pos3: np.ndarray, head_dim: int, split, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Frame-aware RoPE angles: pos3 [T, 3] = (row, col, frame); ``split`` gives the
    channels of each axis (three even numbers summing to d), in axis order row, col, frame.
    Each axis rotates its own contiguous block of channels with its own frequency ladder."""
    split = [int(s) for s in split]
    if len(split) != 3 or sum(split) != head_dim or any(s % 2 for s in split):
        raise ValueError("split must be three even channel counts summing to head_dim")
    pos3 = np.asarray(pos3, dtype=np.float64).reshape(-1, 3)
    parts = [pos3[:, a : a + 1] * axis_frequencies(split[a], theta)[None, :] for a in range(3) if split[a]]
    return np.concatenate(parts, axis=1)


def rope3d(x: np.ndarray, pos3: np.ndarray, split, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Apply frame-aware (row, col, frame) RoPE to x [T, H, d]."""
    x = np.asarray(x, dtype=np.float64)
    return _rotate_pairs(x, angles_3d(pos3, x.shape[-1], split, theta))


def rope3d_inverse(x: np.ndarray, pos3: np.ndarray, split, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Transpose (= inverse) of ``rope3d``: rotation by the negated angles."""
    x = np.asarray(x, dtype=np.float64)
    return _rotate_pairs(x, -angles_3d(pos3, x.shape[-1], split, theta))
