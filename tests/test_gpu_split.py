"""GPU parity of the split last round of the forward.

When the last round of (query tile, head) units fills less of the GPU than a
split would recover, those units are cut into key ranges whose partial results
a merge kernel combines (long samples, more units than compute units). These
batches are built so that the plan splits (the shapes and head counts below
give a short last round of long units on a 256-CU MI355X); outputs and the row
log-sum-exp (also formed by the merge) are checked against the fp64 oracle with
the bars of the whole-unit path, and repeated calls must agree bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_common import check_close, device_inputs, to_f64
from oracle import attention
from text_image_diffusion_varlen_amd import binding, workloads

pytestmark = pytest.mark.gpu

LSE_TOL = 4e-3  # the forward normalizes by a sum of bf16 P (ln(1 + 2^-8)), as in the backward tests

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
    assert np.abs(lse.double().cpu().numpy() - lse_ref).max() <= LSE_TOL
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
    assert np.abs(lse.double().cpu().numpy() - lse_ref).max() <= LSE_TOL
