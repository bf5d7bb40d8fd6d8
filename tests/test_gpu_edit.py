"""GPU parity of the frame-aware (editing) variant: 3D metadata (bit-exact),
frame-aware RoPE, forward, LSE and backward against the fp64 oracle.

Bars as for the 2D path: bf16 forward max abs <= 2e-2 and mean abs <= 2e-3,
fp32 <= 1e-5; RoPE fp32 <= 2e-6 * max|x| and bf16 within one bf16 rounding of
the oracle; gradients as in test_gpu_backward (relative to their own scale).
"""
import numpy as np
import pytest
import torch

from oracle import attention, packing, rope
from text_image_diffusion_varlen_amd import binding, workloads

from gpu_common import TORCH_DTYPE, check_close, check_lse, to_f64

pytestmark = pytest.mark.gpu
GRAD_TOL, GRAD_FLOOR = (2e-2, 1e-2), 1e-5


def _dev(w):
    dt = TORCH_DTYPE[w.dtype]
    q, k, v = (torch.from_numpy(x).to(dt).cuda() for x in (w.q, w.k, w.v))
    grid = torch.from_numpy(w.grid_hw).cuda()
    text = torch.from_numpy(w.text_len).cuda()
    frames = torch.from_numpy(w.frames).cuda()
    return q, k, v, grid, text, frames


def _forward(w, lse=True):
    q, k, v, grid, text, frames = _dev(w)
    cu, _, _ = binding.build_metadata_3d(grid, text, frames, w.tokens)
    res = binding.attn_packed_3d(q, k, v, cu, grid, text, frames, w.rope_split, lse=lse)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    return res


@pytest.mark.parametrize("config", ["edit1024", "edit_mixed"])
def test_metadata_3d_bit_exact(config):
    w = workloads.make_edit(config, heads=1)
    q, k, v, grid, text, frames = _dev(w)
    cu, pos, seg = binding.build_metadata_3d(grid, text, frames, w.tokens)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK
    p_o, s_o = packing.token_positions_3d(w.grid_hw, w.text_len, w.frames)
    assert np.array_equal(cu.cpu().numpy(), packing.cu_seqlens(w.grid_hw, w.text_len, w.frames))
    assert np.array_equal(pos.cpu().numpy(), p_o)
    assert np.array_equal(seg.cpu().numpy(), s_o)


def test_metadata_3d_flags_bad_frames():
    grid = torch.tensor([[2, 2], [3, 1]], dtype=torch.int32, device="cuda")
    text = torch.tensor([1, 2], dtype=torch.int32, device="cuda")
    for fr in ([0, 1], [1, 513]):
        frames = torch.tensor(fr, dtype=torch.int32, device="cuda")
        binding.build_metadata_3d(grid, text, frames, 64)
        assert binding.get_device_error() == binding.MF_ERR_METADATA


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d,split", [(128, (48, 48, 32)), (64, (24, 24, 16)), (128, (64, 32, 32)), (64, (0, 32, 32))])
def test_rope_3d(dtype, d, split):
    rng = np.random.default_rng(60)
    T, H = 300, 3
    x = rng.standard_normal((T, H, d), dtype=np.float32)
    if dtype == "bf16":
        x = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x))
    pos = rng.integers(0, 512, size=(T, 3)).astype(np.int32)
    xt = torch.from_numpy(x).to(TORCH_DTYPE[dtype]).cuda()
    got = binding.rope_3d(xt, torch.from_numpy(pos).cuda(), split)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK
    exp = rope.rope3d(x, pos, split)
    err = np.abs(to_f64(got) - exp)
    if dtype == "f32":
        assert err.max() <= 2e-6 * np.abs(x).max()
    else:
        assert np.all(err <= np.abs(exp) * 2.0 ** -8 + 1e-6)


EDGE = {
    "one_token_images": ([[1, 1], [1, 1]], [0, 3], [1, 4]),
    "thin": ([[1, 5], [5, 1]], [2, 0], [3, 2]),
    "tile_edges": ([[2, 16], [1, 63], [3, 43]], [0, 1, 0], [2, 1, 3]),
    "many_frames": ([[2, 3]], [5], [40]),
}


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_attention_3d_edge_cases(name, dtype, d):
    grid, text, frames = EDGE[name]
    w = workloads.make_edit(grids=grid, texts=text, frames=frames, heads=3, head_dim=d, dtype=dtype, seed=61,
                            scale=1.0 if dtype == "bf16" else 0.125, name=name)
    out, lse = _forward(w)
    exp = attention.joint_attention_3d(w.q, w.k, w.v, w.grid_hw, w.text_len, w.frames, w.rope_split)
    check_close(to_f64(out), exp, dtype)
    ref_lse = attention.joint_attention_3d_lse(w.q, w.k, w.grid_hw, w.text_len, w.frames, w.rope_split)
    if dtype == "bf16":
        check_lse(lse.cpu().numpy(), ref_lse, w)
    else:
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-5


@pytest.mark.parametrize("config", ["edit1024", "edit_mixed"])
def test_attention_3d_configs_two_heads(config):
    w = workloads.make_edit(config, heads=2)
    print(f"edit {config} T={w.tokens}", flush=True)
    out = _forward(w, lse=False)
    exp = attention.joint_attention_3d(w.q, w.k, w.v, w.grid_hw, w.text_len, w.frames, w.rope_split)
    check_close(to_f64(out), exp, w.dtype)


def test_attention_3d_reduces_to_2d_bitwise():
    """frames = 1 and split (d/2, d/2, 0): the same cos/sin values and the same
    arithmetic as the 2D path, so the same output bits."""
    g, t = workloads.make_segments("mixed", seed=25)
    w = workloads.make_edit(grids=g.tolist(), texts=t.tolist(), frames=[1] * len(t), heads=4, head_dim=128,
                            dtype="bf16", seed=62, split=(64, 64, 0))
    q, k, v, grid, text, frames = _dev(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    a = binding.attn_packed(q, k, v, cu, grid, text)
    b = binding.attn_packed_3d(q, k, v, cu, grid, text, frames, (64, 64, 0))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_attention_3d_source_frames_matter():
    """Swapping the source and target images of an edit changes the output
    (the frame index is encoded), while the same data at the same frames is
    reproduced exactly."""
    w = workloads.make_edit(grids=[[4, 4]], texts=[3], frames=[2], heads=2, head_dim=128, dtype="bf16", seed=63)
    out1 = _forward(w, lse=False)
    out2 = _forward(w, lse=False)
    assert torch.equal(out1, out2)
    perm = np.concatenate([np.arange(3), np.arange(19, 35), np.arange(3, 19)])
    ws = workloads.Workload("swap", w.grid_hw, w.text_len, w.heads, w.head_dim, w.dtype, w.q[perm], w.k[perm],
                            w.v[perm], w.seed, w.frames, w.rope_split)
    out3 = _forward(ws, lse=False)
    assert not torch.equal(out3[torch.from_numpy(np.argsort(perm)).cuda()], out1)


def _check_grad(name, got, ref):
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), name
    assert err.max() <= GRAD_TOL[0] * np.abs(ref).max() + GRAD_FLOOR, name
    assert err.mean() <= GRAD_TOL[1] * np.abs(ref).mean() + GRAD_FLOOR, name


@pytest.mark.parametrize("case", ["thin", "tile_edges", "many_frames", "edit_mixed"])
def test_backward_3d(case):
    if case == "edit_mixed":
        w = workloads.make_edit("edit_mixed", heads=2)
    else:
        grid, text, frames = EDGE[case]
        w = workloads.make_edit(grids=grid, texts=text, frames=frames, heads=3, head_dim=128, dtype="bf16", seed=64)
    rng = np.random.default_rng(65)
    do = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal(w.q.shape, dtype=np.float32)))
    q, k, v, grid, text, frames = _dev(w)
    cu, _, _ = binding.build_metadata_3d(grid, text, frames, w.tokens)
    out, lse = binding.attn_packed_3d(q, k, v, cu, grid, text, frames, w.rope_split, lse=True)
    dot = torch.from_numpy(do).to(torch.bfloat16).cuda()
    dq, dk, dv = binding.attn_packed_3d_bwd(q, k, v, out, dot, lse, cu, grid, text, frames, w.rope_split)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    rq, rk, rv = attention.joint_attention_3d_backward(w.q, w.k, w.v, do, w.grid_hw, w.text_len, w.frames,
                                                       w.rope_split)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check_grad(name, to_f64(g), r)


def _heads(w, sel):
    return workloads.Workload(f"{w.name}[heads {sel}]", w.grid_hw, w.text_len, len(sel), w.head_dim, w.dtype,
                              w.q[:, sel], w.k[:, sel], w.v[:, sel], w.seed, w.frames, w.rope_split)


# The editing batches at their real 24 heads: edit1024 (one 8448-token
# sequence, 66 query tiles per head) fills the chip in a few rounds of units
# and takes the split last round; both run the XCD-aware unit order that the
# two- and three-head cases never reach. Heads are independent, so a few of
# them are compared with the oracle run on those head slices alone.
EDIT_ALL_HEADS = {"edit1024": [0, 7, 8, 23], "edit_mixed": [0, 9, 16, 23]}


@pytest.mark.parametrize("config", sorted(EDIT_ALL_HEADS))
def test_attention_3d_configs_all_heads(config):
    w = workloads.make_edit(config)
    sel = EDIT_ALL_HEADS[config]
    print(f"edit {config} T={w.tokens} H={w.heads} compared heads {sel}", flush=True)
    out, lse = _forward(w)
    ws = _heads(w, sel)
    exp = attention.joint_attention_3d(ws.q, ws.k, ws.v, ws.grid_hw, ws.text_len, ws.frames, ws.rope_split)
    check_close(to_f64(out[:, sel]), exp, w.dtype)
    ref_lse = attention.joint_attention_3d_lse(ws.q, ws.k, ws.grid_hw, ws.text_len, ws.frames, ws.rope_split)
    check_lse(lse.cpu().numpy()[sel], ref_lse, ws)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("config,sel", [("edit1024", [0, 8, 23]), ("edit_mixed", [9, 16])])
def test_backward_3d_configs_all_heads(config, sel):
    w = workloads.make_edit(config)
    print(f"edit backward {config} T={w.tokens} H={w.heads} compared heads {sel}", flush=True)
    rng = np.random.default_rng(66)
    do = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal(w.q.shape, dtype=np.float32)))
    q, k, v, grid, text, frames = _dev(w)
    cu, _, _ = binding.build_metadata_3d(grid, text, frames, w.tokens)
    out, lse = binding.attn_packed_3d(q, k, v, cu, grid, text, frames, w.rope_split, lse=True)
    dot = torch.from_numpy(do).to(torch.bfloat16).cuda()
    dq, dk, dv = binding.attn_packed_3d_bwd(q, k, v, out, dot, lse, cu, grid, text, frames, w.rope_split)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    ws = _heads(w, sel)
    rq, rk, rv = attention.joint_attention_3d_backward(ws.q, ws.k, ws.v, do[:, sel], ws.grid_hw, ws.text_len,
                                                       ws.frames, ws.rope_split)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check_grad(name, to_f64(g[:, sel]), r)
        assert torch.isfinite(g.float()).all(), f"{name}: non-finite"


def test_attention_3d_rejects_bad_split():
    w = workloads.make_edit(grids=[[2, 2]], texts=[1], frames=[2], heads=1, head_dim=64, dtype="bf16", seed=1)
    q, k, v, grid, text, frames = _dev(w)
    cu, _, _ = binding.build_metadata_3d(grid, text, frames, w.tokens)
    for split in ((30, 30, 2), (31, 31, 2), (64, 0, 2)):
        with pytest.raises(binding.MFError) as e:
            binding.attn_packed_3d(q, k, v, cu, grid, text, frames, split)
        assert e.value.code == binding.MF_ERR_INVALID_ARG
