"""Helpers shared by the GPU tests: move seeded workloads to the device, run
the library through its C ABI, and the parity bars. No arithmetic of the
method lives here (the LSE bar's operand bound uses the oracle's rotation)."""
import math

import numpy as np
import torch

from text_image_diffusion_varlen_amd import binding

TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-5)}  # (max abs, mean abs) vs the fp64 oracle
TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def device_inputs(w, dev="cuda"):
    dt = TORCH_DTYPE[w.dtype]
    q, k, v = (torch.from_numpy(x).to(dt).to(dev) for x in (w.q, w.k, w.v))
    grid = torch.from_numpy(w.grid_hw).to(dev)
    text = torch.from_numpy(w.text_len).to(dev)
    return q, k, v, grid, text


def run_attention(w, out=None):
    """Runs the whole path on the GPU; cu_seqlens comes from the library's own metadata builder."""
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    out = binding.attn_packed(q, k, v, cu, grid, text, out=out)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    return out


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_close(got, exp, dtype):
    max_tol, mean_tol = TOL[dtype]
    err = np.abs(got - exp)
    assert np.isfinite(got).all(), "non-finite output"
    assert err.max() <= max_tol and err.mean() <= mean_tol, (
        f"max abs {err.max():.3e} (tol {max_tol}), mean abs {err.mean():.3e} (tol {mean_tol})")
    return float(err.max()), float(err.mean())


U_BF16 = 2.0 ** -8                 # unit roundoff of bf16 (8 significant bits)
LSE_P_TERM = math.log1p(U_BF16)    # the forward normalizes by a sum of bf16-rounded P


def check_lse(got, ref, w):
    """Row log-sum-exp [H][T] of a bf16 forward against the fp64 oracle.

    Per row the bar is ln(1 + u) + scale (2u + u^2 + d 2^-24) max_i sum_j |q~_j k~_ij| + 1e-5
    (u = 2^-8): the first term bounds the relative error of the row sum of bf16
    P the forward divides by; the second bounds how far the bf16 rounding of
    the rotated operands Q~ and K~ (and fp32 accumulation over d) can move any
    scaled score, and the log-sum-exp moves by at most the largest score shift.
    Long rows average the second term away; rows of a few keys do not. It is
    evaluated (with the oracle's rotation) only for rows above the first term.
    Returns the largest error."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), "non-finite LSE"
    err = np.abs(got - ref)
    hot = np.argwhere(err > LSE_P_TERM + 1e-5)
    if hot.size:
        from oracle import packing, rope
        frames = getattr(w, "frames", None)
        cu = packing.cu_seqlens(w.grid_hw, w.text_len, frames)
        if frames is None:
            pos, _ = packing.token_positions(w.grid_hw, w.text_len)
            qr, kr = rope.rope2d(w.q, pos), rope.rope2d(w.k, pos)
        else:
            pos3, _ = packing.token_positions_3d(w.grid_hw, w.text_len, frames)
            qr, kr = rope.rope3d(w.q, pos3, w.rope_split), rope.rope3d(w.k, pos3, w.rope_split)
        d = w.head_dim
        coef = (2 * U_BF16 + U_BF16 * U_BF16 + d * 2.0 ** -24) / math.sqrt(d)
        for h, t in hot:
            s = int(np.searchsorted(cu, t, side="right")) - 1
            a, b = int(cu[s]), int(cu[s + 1])
            shift = coef * float((np.abs(kr[a:b, h]) @ np.abs(qr[t, h])).max())
            bound = LSE_P_TERM + shift + 1e-5
            assert err[h, t] <= bound, f"LSE row (head {h}, token {t}): err {err[h, t]:.3e} > bound {bound:.3e}"
    return float(err.max())
