"""Rectified flow (oracle, fp64).

TEST INFRASTRUCTURE: used only by tests, the smoke check and the CPU baseline.

Source: mageflow.net architecture page, section 3 ("Rectified Flow Matching
Trajectories"): noise z_0 ~ N(0, I) and data z_1 are joined by straight
paths z_t = t z_1 + (1 - t) z_0 with constant velocity z_1 - z_0; the model
v_theta is trained to that velocity with a squared-error loss and sampled
with Euler or midpoint steps. The tech report's own equation for this
objective did not survive extraction; section 3's convention (t = 0 is noise,
t = 1 is data) is the one used here.

Classifier-free guidance (packed conditional and unconditional branches,
tech report NR-MMDiT section) combines the two velocities; the pages do not
print the combination, the standard one v_u + s (v_c - v_u) is taken.
"""
from __future__ import annotations

import numpy as np

from .packing import cu_seqlens


def interpolate(z0, z1, t):
    """z_t = t * z_1 + (1 - t) * z_0."""
    z0 = np.asarray(z0, dtype=np.float64)
    z1 = np.asarray(z1, dtype=np.float64)
    return t * z1 + (1.0 - t) * z0


def target_velocity(z0, z1):
    """v = z_1 - z_0 (constant along the straight path)."""
    return np.asarray(z1, dtype=np.float64) - np.asarray(z0, dtype=np.float64)


def loss(v_pred, z0, z1) -> float:
    """Mean over samples (leading axis) of the squared norm || v_pred - (z_1 - z_0) ||^2."""
    r = np.asarray(v_pred, dtype=np.float64) - target_velocity(z0, z1)
    r = r.reshape(r.shape[0], -1)
    return float(np.mean(np.sum(r * r, axis=1)))


def euler(z, velocity, t_grid):
    """Explicit Euler: z <- z + (t_{k+1} - t_k) * v(z, t_k) over the time grid.
    Returns the list of states at every grid point (first entry = input)."""
    z = np.asarray(z, dtype=np.float64)
    states = [z]
    for k in range(len(t_grid) - 1):
        dt = t_grid[k + 1] - t_grid[k]
        z = z + dt * velocity(z, t_grid[k])
        states.append(z)
    return states


def midpoint(z, velocity, t_grid):
    """Explicit midpoint: z_mid = z + dt/2 * v(z, t_k); z <- z + dt * v(z_mid, t_k + dt/2)."""
    z = np.asarray(z, dtype=np.float64)
    states = [z]
    for k in range(len(t_grid) - 1):
        t = t_grid[k]
        dt = t_grid[k + 1] - t
        z_mid = z + 0.5 * dt * velocity(z, t)
        z = z + dt * velocity(z_mid, t + 0.5 * dt)
        states.append(z)
    return states


def uniform_grid(steps: int):
    """t_k = k / steps, k = 0 .. steps (no time shift: the pages print none)."""
    return [k / steps for k in range(steps + 1)]


def cfg_combine(v_uncond, v_cond, guidance: float):
    """Guided velocity v_u + s * (v_c - v_u)."""
    vu = np.asarray(v_uncond, dtype=np.float64)
    vc = np.asarray(v_cond, dtype=np.float64)
    return vu + guidance * (vc - vu)


def packed_cfg_euler_step(z, v, grid_hw, text_len, cond_seg, uncond_seg, guidance: float, dt: float):
    """One guided Euler step for every image of a packed CFG batch.

    The batch packs samples [prompt; h*w image tokens] back to back (tech report,
    NR-MMDiT section: conditional and unconditional branches in one pass).
    Image b's conditional velocities are the image rows of sample cond_seg[b],
    its unconditional ones those of uncond_seg[b] (or the conditional ones when
    that is -1). z holds the images' tokens back to back in image order; each
    image moves by dt * cfg_combine(v_u, v_c, guidance).
    """
    grid_hw = np.asarray(grid_hw).reshape(-1, 2)
    text_len = np.asarray(text_len)
    v = np.asarray(v, dtype=np.float64)
    cu = cu_seqlens(grid_hw, text_len)
    out = np.array(z, dtype=np.float64)
    start = 0
    for b in range(len(cond_seg)):
        cs, us = int(cond_seg[b]), int(uncond_seg[b])
        n = int(grid_hw[cs, 0]) * int(grid_hw[cs, 1])
        vc = v[cu[cs] + text_len[cs]: cu[cs + 1]]
        vu = vc if us < 0 else v[cu[us] + text_len[us]: cu[us + 1]]
        out[start:start + n] += dt * cfg_combine(vu, vc, guidance)
        start += n
    return out
