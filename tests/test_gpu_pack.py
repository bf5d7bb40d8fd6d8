"""GPU parity of the joint-layout pack and unpack (mf_pack_joint,
mf_unpack_joint) against the oracle's pack_joint / unpack_joint.

Pure copies, so the bar is bit-exact: every byte of every output equals the
oracle's. The streams are seeded bf16 / fp32 values of the workloads' shapes;
q, k and v move in one launch. Also: the round trip returns the streams, a
mismatched cu_seqlens (or prompt total) writes nothing and is flagged, and
editing samples (several images per sample) pack their images one after
another.
"""
import numpy as np
import pytest
import torch

from oracle import packing
from text_image_diffusion_varlen_amd import binding, workloads

pytestmark = pytest.mark.gpu
TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def _streams(grid, text, frames, heads, d, dtype, seed, n_tensors=3):
    rng = np.random.default_rng(seed)
    f = 1 if frames is None else np.asarray(frames)
    n_text = int(np.sum(text))
    n_img = int(np.sum(f * np.asarray(grid)[:, 0] * np.asarray(grid)[:, 1]))
    out = []
    for _ in range(n_tensors):
        ts = rng.standard_normal((n_text, heads, d), dtype=np.float32)
        im = rng.standard_normal((n_img, heads, d), dtype=np.float32)
        if dtype == "bf16":
            ts = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(ts))
            im = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(im))
        out.append((ts, im))
    return out


def _dev(x, dtype):
    return torch.from_numpy(x).to(TORCH[dtype]).cuda()


def _check(grid, text, frames, heads, d, dtype, seed, n_tensors=3):
    grid = np.asarray(grid, dtype=np.int32).reshape(-1, 2)
    text = np.asarray(text, dtype=np.int32)
    fr = None if frames is None else np.asarray(frames, dtype=np.int32)
    streams = _streams(grid, text, fr, heads, d, dtype, seed, n_tensors)
    g, t = torch.from_numpy(grid).cuda(), torch.from_numpy(text).cuda()
    fd = None if fr is None else torch.from_numpy(fr).cuda()
    cu = torch.from_numpy(packing.cu_seqlens(grid, text, fr)).cuda()
    text_t = [_dev(s[0], dtype) for s in streams]
    img_t = [_dev(s[1], dtype) for s in streams]
    joint = binding.pack_joint(text_t, img_t, cu, g, t, frames=fd)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    for (ts, im), j in zip(streams, joint):
        exp = packing.pack_joint(ts, im, grid, text, fr)
        assert torch.equal(j.cpu(), torch.from_numpy(exp).to(TORCH[dtype])), "joint rows differ from the oracle"
    back_t, back_i = binding.unpack_joint(joint, int(text.sum()), cu, g, t, frames=fd)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    for (ts, im), j, bt, bi in zip(streams, joint, back_t, back_i):
        et, ei = packing.unpack_joint(j.cpu().float().numpy(), grid, text, fr)
        assert torch.equal(bt.cpu(), torch.from_numpy(et).to(TORCH[dtype]))
        assert torch.equal(bi.cpu(), torch.from_numpy(ei).to(TORCH[dtype]))
        assert torch.equal(bt.cpu(), torch.from_numpy(ts).to(TORCH[dtype])), "round trip (text)"
        assert torch.equal(bi.cpu(), torch.from_numpy(im).to(TORCH[dtype])), "round trip (image)"


@pytest.mark.parametrize("config", ["1024sq", "mixed", "train65k"])
def test_pack_configs(config):
    grid, text = workloads.make_segments(config)
    print(f"pack {config}: {len(text)} samples", flush=True)
    _check(grid, text, None, 24, 128, "bf16", seed=1)


def test_pack_edit_frames():
    _check([[32, 128], [64, 64], [48, 84]], [100, 77, 256], [2, 3, 2], 24, 128, "bf16", seed=2)


EDGE = {
    "no_prompts": ([[3, 5], [1, 1], [7, 2]], [0, 0, 0]),
    "one_token": ([[1, 1]], [0]),
    "prompt_heavy": ([[1, 1], [2, 2]], [300, 1]),
    "many": (np.random.default_rng(5).integers(1, 4, size=(4096, 2)).tolist(),
             np.random.default_rng(6).integers(0, 3, size=4096).tolist()),
}


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("dtype,d,heads", [("bf16", 128, 3), ("f32", 64, 2), ("bf16", 64, 1)])
def test_pack_edge_cases(name, dtype, d, heads):
    grid, text = EDGE[name]
    _check(grid, text, None, heads, d, dtype, seed=7, n_tensors=2)


def test_pack_single_tensor_and_four_tensors():
    _check([[4, 6], [2, 9]], [5, 11], None, 8, 128, "bf16", seed=8, n_tensors=1)
    _check([[4, 6], [2, 9]], [5, 11], None, 8, 128, "bf16", seed=9, n_tensors=4)


def test_pack_metadata_mismatch_writes_nothing():
    grid = torch.tensor([[4, 4], [3, 5]], dtype=torch.int32, device="cuda")
    text = torch.tensor([2, 1], dtype=torch.int32, device="cuda")
    T = 2 + 16 + 1 + 15
    ts = [torch.ones((3, 2, 128), dtype=torch.bfloat16, device="cuda")]
    im = [torch.ones((31, 2, 128), dtype=torch.bfloat16, device="cuda")]
    out = [torch.full((T, 2, 128), 5.0, dtype=torch.bfloat16, device="cuda")]
    bad_cu = torch.tensor([0, 17, T], dtype=torch.int32, device="cuda")
    binding.pack_joint(ts, im, bad_cu, grid, text, out=out)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    assert torch.all(out[0] == 5.0)
    # prompt total that disagrees with the text stream's length
    cu = torch.tensor([0, 18, T], dtype=torch.int32, device="cuda")
    binding.unpack_joint(out, 4, cu, grid, text, out=([torch.zeros((4, 2, 128), dtype=torch.bfloat16,
                                                                    device="cuda")],
                                                       [torch.zeros((30, 2, 128), dtype=torch.bfloat16,
                                                                    device="cuda")]))
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    binding.pack_joint(ts, im, cu, grid, text, out=out)  # consistent: succeeds
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    assert torch.all(out[0] == 1.0)
