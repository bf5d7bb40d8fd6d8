"""GPU parity of the metadata builder (bit-exact) and of the 2D RoPE kernel."""
import numpy as np
import pytest
import torch

from oracle import packing, rope
from text_image_diffusion_varlen_amd import binding, workloads

from gpu_common import device_inputs

pytestmark = pytest.mark.gpu


def _meta_case(grid, text):
    grid_d = torch.tensor(np.asarray(grid, np.int32).reshape(-1, 2), device="cuda")
    text_d = torch.tensor(np.asarray(text, np.int32), device="cuda")
    T = int(packing.cu_seqlens(grid, text)[-1])
    cu, pos, seg = binding.build_metadata(grid_d, text_d, T)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK
    cu_o = packing.cu_seqlens(grid, text)
    pos_o, seg_o = packing.token_positions(grid, text)
    assert np.array_equal(cu.cpu().numpy(), cu_o)
    assert np.array_equal(pos.cpu().numpy(), pos_o)
    assert np.array_equal(seg.cpu().numpy(), seg_o)


@pytest.mark.parametrize("config", ["tiny", "1024sq", "mixed", "2048sq", "train65k"])
def test_metadata_configs_bit_exact(config):
    print(f"metadata {config}", flush=True)
    grid, text = workloads.make_segments(config)
    _meta_case(grid, text)


def test_metadata_edge_cases_bit_exact():
    cases = [
        ([[1, 1]], [0]),
        ([[1, 1]], [5]),
        ([[512, 512]], [0]),
        ([[1, 512], [512, 1], [3, 7]], [0, 1, 300]),
        ([[2, 3], [1, 2], [3, 1]], [2, 0, 1]),
    ]
    rng = np.random.default_rng(7)
    for _ in range(4):
        n = int(rng.integers(1, 300))
        cases.append((rng.integers(1, 40, size=(n, 2)).tolist(), rng.integers(0, 80, size=n).tolist()))
    # 64 / 65 samples (the one-wave path and the workgroup path) and the maximum, 4096
    for n in (64, 65, 4096):
        cases.append((rng.integers(1, 4, size=(n, 2)).tolist(), rng.integers(0, 4, size=n).tolist()))
    for grid, text in cases:
        _meta_case(grid, text)


def test_metadata_flags_bad_inputs():
    grid = torch.tensor([[4, 4], [0, 3]], dtype=torch.int32, device="cuda")
    text = torch.tensor([2, 2], dtype=torch.int32, device="cuda")
    binding.build_metadata(grid, text, 24)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    # wrong capacity: flagged, nothing written past it
    grid = torch.tensor([[4, 4]], dtype=torch.int32, device="cuda")
    text = torch.tensor([2], dtype=torch.int32, device="cuda")
    binding.build_metadata(grid, text, 17)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    # the flag is sticky until read, then clear
    _meta_case([[4, 4]], [2])


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_rope_matches_oracle(dtype, d):
    w = workloads.make_custom([[20, 30], [7, 3]], [11, 0], heads=3, head_dim=d, dtype=dtype, seed=3)
    pos, _ = packing.token_positions(w.grid_hw, w.text_len)
    # also exercise the far end of the table
    pos[-1] = [511, 511]
    pos[-2] = [0, 511]
    q, _, _, _, _ = device_inputs(w)
    got = binding.rope_2d(q, torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK
    exp = rope.rope2d(w.q.astype(np.float64), pos)
    g = got.float().cpu().numpy().astype(np.float64)
    if dtype == "f32":
        np.testing.assert_allclose(g, exp, rtol=0, atol=2e-6 * np.abs(w.q).max())
    else:
        # fp32 math then one bf16 rounding: within one bf16 ulp of the exact value
        # (plus an absolute fp32 slack where the rotation cancels to near zero)
        bound = np.abs(exp) * 2.0 ** -7 + 2e-6 * np.abs(w.q).max()
        assert np.all(np.abs(g - exp) <= bound)


def test_rope_relative_position_invariance_on_gpu():
    """q~ . k~ through the GPU kernel depends only on the position difference."""
    rng = np.random.default_rng(4)
    T, H, d = 64, 2, 128
    q = torch.from_numpy(rng.standard_normal((T, H, d), dtype=np.float32)).cuda()
    k = torch.from_numpy(rng.standard_normal((T, H, d), dtype=np.float32)).cuda()
    pq = rng.integers(0, 200, size=(T, 2)).astype(np.int32)
    pk = rng.integers(0, 200, size=(T, 2)).astype(np.int32)

    def dots(shift):
        a = binding.rope_2d(q, torch.from_numpy(pq + shift).cuda())
        b = binding.rope_2d(k, torch.from_numpy(pk + shift).cuda())
        a = a.cpu().numpy().astype(np.float64)
        b = b.cpu().numpy().astype(np.float64)
        return np.einsum("thd,shd->tsh", a, b)

    base = dots(np.array([0, 0], np.int32))
    for shift in ([3, 0], [0, 50], [100, 100]):
        np.testing.assert_allclose(dots(np.array(shift, np.int32)), base, atol=2e-3)


def test_rope_flags_out_of_range_positions():
    x = torch.ones((2, 1, 64), dtype=torch.float32, device="cuda")
    pos = torch.tensor([[0, 0], [512, 0]], dtype=torch.int32, device="cuda")
    y = binding.rope_2d(x, pos)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    assert torch.equal(y[1], x[1])
