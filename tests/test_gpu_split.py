"""GPU parity of the split last round (forward, and the backward's dK/dV and dQ kernels).

When the last round of work units fills less of the GPU than a split would
recover, those units are cut into pieces whose partial results a merge kernel
combines: forward and dQ units (query tile, head) over key ranges, dK/dV
units (128-key block, head) over query ranges. These batches are built so that the
plans split (the shapes and head counts below give a short last round of long
units on a 256-CU MI355X); outputs, the row log-sum-exp (formed by the forward
merge) and the gradients are checked against the fp64 oracle with the bars of
the whole-unit paths, and repeated calls must agree bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_common import check_close, check_lse, device_inputs, to_f64
from oracle import attention
from text_image_diffusion_varlen_amd import binding, workloads

pytestmark = pytest.mark.gpu


# name: (grids, prompt lengths, heads, head_dim)
SPLIT_2D = {
    # one 9000-token sample, 8 heads: 288 units, the last 32 in a 4-way split
    "one_long_d128": ([[88, 100]], [200], 8, 128),
    "one_long_d64": ([[88, 100]], [200], 8, 64),
    # two long samples, 4 heads: 284 units, the last 28 (the shorter sample's) split
    "two_long": ([[96, 100], [90, 92]], [77, 150], 4, 128),
}


def _forward(q, k, v, grid, text, cu, frames=None, split=None):
    if frames is None:
        out, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
    else:
        out, lse = binding.attn_packed_3d(q, k, v, cu, grid, text, frames, split, lse=True)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    return out, lse


@pytest.mark.parametrize("name", sorted(SPLIT_2D))
def test_split_round_2d(name):
    grids, texts, heads, d = SPLIT_2D[name]
    w = workloads.make_custom(grids, texts, heads=heads, head_dim=d, dtype="bf16", seed=17, name=name)
    print(f"split {name} T={w.tokens} n={w.n_seg} H={heads} d={d}", flush=True)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    out, lse = _forward(q, k, v, grid, text, cu)
    check_close(to_f64(out), attention.joint_attention(w.q, w.k, w.v, w.grid_hw, w.text_len), "bf16")
    lse_ref = attention.joint_attention_lse(w.q, w.k, w.grid_hw, w.text_len)
    check_lse(lse.double().cpu().numpy(), lse_ref, w)
    out2, lse2 = _forward(q, k, v, grid, text, cu)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "repeated calls differ"


def test_split_round_16_heads_partly_split_sample():
    """One 9000-token sample with 16 heads: 576 units, the last 64 split 4 ways.
    Heads are a multiple of 8, so the whole units take the XCD-aware head-major
    order; the sample's last 4 query tiles are split, so the order covers only
    its first 32 tiles (the partly split branch of the unit permutation).
    Output and LSE of six heads, every element, against the oracle on those
    head slices (heads are independent)."""
    sel = [0, 3, 7, 8, 12, 15]
    w = workloads.make_custom([[88, 100]], [200], heads=16, head_dim=128, dtype="bf16", seed=19, name="h16")
    print(f"split 16 heads T={w.tokens} compared heads {sel}", flush=True)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    out, lse = _forward(q, k, v, grid, text, cu)
    ws = workloads.Workload("h16 subset", w.grid_hw, w.text_len, len(sel), w.head_dim, w.dtype,
                            w.q[:, sel], w.k[:, sel], w.v[:, sel], seed=w.seed)
    check_close(to_f64(out[:, sel]), attention.joint_attention(ws.q, ws.k, ws.v, ws.grid_hw, ws.text_len), "bf16")
    lse_ref = attention.joint_attention_lse(ws.q, ws.k, ws.grid_hw, ws.text_len)
    check_lse(lse.double().cpu().numpy()[sel], lse_ref, ws)
    assert torch.isfinite(out.float()).all()
    out2, lse2 = _forward(q, k, v, grid, text, cu)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), "repeated calls differ"


def test_split_round_edit():
    # one edit of 3 images of 48 x 64 after a 100-token instruction, 8 heads: 296 units, 40 split
    w = workloads.make_edit(grids=[[48, 64]], texts=[100], frames=[3], heads=8, head_dim=128, dtype="bf16",
                            seed=18, split=workloads.EDIT_SPLIT[128], name="split_edit")
    print(f"split edit T={w.tokens} H={w.heads}", flush=True)
    q, k, v, grid, text = device_inputs(w)
    frames = torch.from_numpy(w.frames).cuda()
    cu, _, _ = binding.build_metadata_3d(grid, text, frames, w.tokens)
    out, lse = _forward(q, k, v, grid, text, cu, frames, w.rope_split)
    ref = attention.joint_attention_3d(w.q, w.k, w.v, w.grid_hw, w.text_len, w.frames, w.rope_split)
    check_close(to_f64(out), ref, "bf16")
    lse_ref = attention.joint_attention_3d_lse(w.q, w.k, w.grid_hw, w.text_len, w.frames, w.rope_split)
    check_lse(lse.double().cpu().numpy(), lse_ref, w)


# Backward: the dK/dV kernel's units are (128-key block, head); a 4352-token
# sample with 8 heads gives 272 units, the last 16 split 4 ways over query ranges.
# The dQ kernel's units are (256-query tile, head) and split over key ranges
# when the mean sample length reaches the forward's threshold: a 9000-token
# sample with 2 heads gives 72 dQ units, all in a partly filled round, split 3
# ways (and 144 dK/dV units, also split).
BWD_SPLIT = {
    "bwd_1024_d128": ([[64, 64]], [256], 8, 128),
    "bwd_1024_d64": ([[64, 64]], [256], 8, 64),
    "bwd_edit": None,  # a 2-image edit of 40 x 52 after a 70-token prompt, 8 heads (frame-aware path)
    "bwd_long_d128": ([[88, 100]], [200], 2, 128),
    "bwd_long_d64": ([[88, 100]], [200], 2, 64),
    "bwd_edit_long": None,  # a 3-image edit of 48 x 64 after a 100-token prompt, 2 heads (dQ split, frame-aware)
}
GRAD_TOL = (2e-2, 1e-2)  # relative to the reference's own max / mean magnitude, as in the backward tests
GRAD_FLOOR = 1e-5


def _check_grad(name, got, ref):
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{name}: non-finite"
    assert err.max() <= GRAD_TOL[0] * np.abs(ref).max() + GRAD_FLOOR, name
    assert err.mean() <= GRAD_TOL[1] * np.abs(ref).mean() + GRAD_FLOOR, name


@pytest.mark.parametrize("name", sorted(BWD_SPLIT))
def test_split_round_backward(name):
    if name == "bwd_edit":
        w = workloads.make_edit(grids=[[40, 52]], texts=[70], frames=[2], heads=8, head_dim=128, dtype="bf16",
                                seed=21, name=name)
    elif name == "bwd_edit_long":
        w = workloads.make_edit(grids=[[48, 64]], texts=[100], frames=[3], heads=2, head_dim=128, dtype="bf16",
                                seed=23, split=workloads.EDIT_SPLIT[128], name=name)
    else:
        grids, texts, heads, d = BWD_SPLIT[name]
        w = workloads.make_custom(grids, texts, heads=heads, head_dim=d, dtype="bf16", seed=20, name=name)
    print(f"split {name} T={w.tokens} H={w.heads} d={w.head_dim}", flush=True)
    rng = np.random.default_rng(22)
    do = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal(w.q.shape, dtype=np.float32)))
    q, k, v, grid, text = device_inputs(w)
    dot = torch.from_numpy(do).to(torch.bfloat16).cuda()
    if w.frames is None:
        cu, _, _ = binding.build_metadata(grid, text, w.tokens)
        out, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
        run = lambda: binding.attn_packed_bwd(q, k, v, out, dot, lse, cu, grid, text)  # noqa: E731
        ref = attention.joint_attention_backward(w.q, w.k, w.v, do, w.grid_hw, w.text_len)
    else:
        frames = torch.from_numpy(w.frames).cuda()
        cu, _, _ = binding.build_metadata_3d(grid, text, frames, w.tokens)
        out, lse = binding.attn_packed_3d(q, k, v, cu, grid, text, frames, w.rope_split, lse=True)
        run = lambda: binding.attn_packed_3d_bwd(q, k, v, out, dot, lse, cu, grid, text, frames,  # noqa: E731
                                                 w.rope_split)
        ref = attention.joint_attention_3d_backward(w.q, w.k, w.v, do, w.grid_hw, w.text_len, w.frames,
                                                    w.rope_split)
    grads = run()
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    for nm, g, r in zip(("dq", "dk", "dv"), grads, ref):
        _check_grad(nm, to_f64(g), r)
    again = run()
    torch.cuda.synchronize()
    for nm, g, g2 in zip(("dq", "dk", "dv"), grads, again):
        assert torch.equal(g, g2), f"{nm}: repeated calls differ"
