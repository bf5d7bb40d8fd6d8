"""Helpers shared by the GPU tests: move seeded workloads to the device and run
the library through its C ABI. No arithmetic of the method lives here."""
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
