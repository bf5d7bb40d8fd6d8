"""Input construction shared by the CPU and GPU tests of the packed CFG step.

Builds velocity fields with a known closed-form trajectory: for every image,
target = (z1 - z) / (1 - t) (the straight rectified-flow path through z), and
the conditional / unconditional velocities are offset by e (1 - 1/s) and e so
that v_u + s (v_c - v_u) = target exactly in exact arithmetic. An Euler step of
size dt then moves z to the straight path's point at t + dt, so four steps of
1/4 land on z1 -- but only if the step gathers the right rows of the packed
batch and combines them with the right sign.
"""
import numpy as np


def sample_starts(batch):
    """First token of every sample, from an explicit running sum."""
    starts, run = [], 0
    for (h, w), t in zip(batch.grid_hw.tolist(), batch.text_len.tolist()):
        starts.append(run)
        run += t + h * w
    return starts


def image_slices(batch):
    """(start, stop) of every image's tokens inside z."""
    out, run = [], 0
    for b in range(batch.n_img):
        h, w = batch.grid_hw[batch.cond_seg[b]].tolist()
        out.append((run, run + h * w))
        run += h * w
    return out


def guided_field(batch, z, z1, t, guidance, noise, dtype=np.float64):
    """Packed velocities [tokens, C] whose guided combination is (z1 - z)/(1 - t).

    Text rows keep ``noise`` (they must not matter). ``noise`` has the shape of
    the packed velocity and supplies e per sample row.
    """
    v = np.array(noise, dtype=np.float64)
    starts = sample_starts(batch)
    for b, (a, c) in enumerate(image_slices(batch)):
        target = (z1[a:c] - z[a:c]) / (1.0 - t)
        cs, us = int(batch.cond_seg[b]), int(batch.uncond_seg[b])
        ci = starts[cs] + int(batch.text_len[cs])
        if us < 0:
            v[ci:ci + (c - a)] = target
            continue
        ui = starts[us] + int(batch.text_len[us])
        e = noise[ui:ui + (c - a)]
        v[ui:ui + (c - a)] = target + e
        v[ci:ci + (c - a)] = target + e * (1.0 - 1.0 / guidance)
    return v.astype(dtype)
