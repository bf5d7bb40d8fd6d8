"""GPU parity of the packed CFG rectified-flow Euler step (mf_rf_cfg_euler_step)
against the fp64 oracle.

z is float32 and the step's arithmetic is fp32, so the bar is the fp32 one:
max abs and mean abs <= 1e-5 against the oracle on the same inputs (values of z
reach ~20 here; fp32 rounds a sum of that size to ~1e-6)."""
import numpy as np
import pytest
import torch

from oracle import packing, rectified_flow
from text_image_diffusion_varlen_amd import binding, workloads

from cfg_common import guided_field
from gpu_common import check_close

pytestmark = pytest.mark.gpu
TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def _device(batch, v=None):
    v = batch.v if v is None else v
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(TORCH_DTYPE[batch.dtype]).cuda()
    cu = torch.from_numpy(packing.cu_seqlens(batch.grid_hw, batch.text_len)).cuda()
    grid = torch.from_numpy(batch.grid_hw).cuda()
    text = torch.from_numpy(batch.text_len).cuda()
    cs = torch.from_numpy(batch.cond_seg).cuda()
    us = torch.from_numpy(batch.uncond_seg).cuda()
    return vt, cu, grid, text, cs, us


def _step(batch, guidance, dt, z=None, v=None):
    z = torch.from_numpy(batch.z).cuda() if z is None else z
    vt, cu, grid, text, cs, us = _device(batch, v)
    binding.rf_cfg_euler_step(z, vt, cu, grid, text, cs, us, guidance, dt)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    return z


def _oracle(batch, guidance, dt, z=None, v=None):
    z = batch.z if z is None else z
    v = batch.v if v is None else v
    return rectified_flow.packed_cfg_euler_step(z, v, batch.grid_hw, batch.text_len, batch.cond_seg,
                                                batch.uncond_seg, guidance, dt)


@pytest.mark.parametrize("config", ["cfg1024", "cfg_mixed"])
@pytest.mark.parametrize("layout", ["interleaved", "blocks", "shuffled"])
def test_cfg_step_configs(config, layout):
    print(f"cfg step {config} {layout}", flush=True)
    batch = workloads.make_cfg_config(config, layout=layout)
    got = _step(batch, 5.0, 0.25).cpu().numpy().astype(np.float64)
    check_close(got, _oracle(batch, 5.0, 0.25), "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("channels", [8, 16, 128, 136])
def test_cfg_step_edge_cases(dtype, channels):
    grids = [(1, 1), (1, 9), (9, 1), (5, 7), (1, 1)]
    batch = workloads.make_cfg_batch(grids, [0, 77, 3, 256, 1], [0, 5, 0, 0, 2], "shuffled", channels, dtype,
                                     seed=channels, guided=[1, 0, 1, 1, 0])
    for s, dt in [(5.0, 0.25), (1.0, 1.0), (0.0, -0.5), (7.5, 1e-3)]:
        got = _step(batch, s, dt).cpu().numpy().astype(np.float64)
        check_close(got, _oracle(batch, s, dt), "f32")


def test_cfg_step_many_images():
    """More images than threads of the offsets kernel, so each thread owns a run of images."""
    rng = np.random.default_rng(40)
    grids = rng.integers(1, 6, size=(1500, 2)).tolist()
    batch = workloads.make_cfg_batch(grids, rng.integers(0, 9, size=1500).tolist(), 0, "blocks", 16, "bf16",
                                     seed=41, guided=(rng.random(1500) < 0.8).tolist())
    got = _step(batch, 4.0, 0.125).cpu().numpy().astype(np.float64)
    check_close(got, _oracle(batch, 4.0, 0.125), "f32")


@pytest.mark.parametrize("guidance", [5.0, 1.0])
def test_cfg_four_step_loop_lands_on_data(guidance):
    """A four-step guided loop along the constructed field follows the straight
    path and lands on z1 (the oracle's closed form), with z kept on the device."""
    batch = workloads.make_cfg_config("cfg_mixed", layout="shuffled")
    batch.dtype = "f32"
    rng = np.random.default_rng(50)
    z0 = batch.z.astype(np.float64)
    z1 = rng.standard_normal(z0.shape)
    z = torch.from_numpy(batch.z).cuda()
    grid = rectified_flow.uniform_grid(4)
    for k in range(4):
        t, dt = grid[k], grid[k + 1] - grid[k]
        zk = z.cpu().numpy().astype(np.float64)
        v = guided_field(batch, zk, z1, t, guidance, rng.standard_normal(batch.v.shape), np.float32)
        _step(batch, guidance, dt, z=z, v=v)
        check_close(z.cpu().numpy().astype(np.float64), grid[k + 1] * z1 + (1 - grid[k + 1]) * z0, "f32")
    check_close(z.cpu().numpy().astype(np.float64), z1, "f32")


def test_cfg_step_second_call_smaller():
    big = workloads.make_cfg_config("cfg1024")
    small = workloads.make_cfg_batch([(3, 3), (2, 5)], [4, 1], [0, 0], "blocks", 128, "bf16", seed=3)
    for b in (big, small, big):
        got = _step(b, 5.0, 0.25).cpu().numpy().astype(np.float64)
        check_close(got, _oracle(b, 5.0, 0.25), "f32")


def _bad_call(batch, **over):
    z = torch.from_numpy(batch.z).cuda()
    z_before = z.clone()
    vt, cu, grid, text, cs, us = _device(batch)
    args = dict(cu=cu, grid=grid, text=text, cs=cs, us=us)
    args.update(over)
    binding.rf_cfg_euler_step(z, vt, args["cu"], args["grid"], args["text"], args["cs"], args["us"], 5.0, 0.25)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    assert torch.equal(z, z_before)


def test_cfg_step_flags_inconsistent_maps_and_writes_nothing():
    batch = workloads.make_cfg_batch([(4, 4), (3, 5)], [2, 3], [0, 1], "interleaved", 8, "bf16", seed=5)
    dev = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")  # noqa: E731
    # unconditional sample of image 0 is image 1's (different grid)
    _bad_call(batch, us=dev([3, 1]))
    # index out of range, and below -1
    _bad_call(batch, cs=dev([0, 4]))
    _bad_call(batch, us=dev([-2, 3]))
    # cu_seqlens that disagrees with the grids and prompts
    cu = packing.cu_seqlens(batch.grid_hw, batch.text_len).copy()
    cu[1] += 1
    _bad_call(batch, cu=dev(cu.tolist()))
    # image_tokens that does not match the grids (z one token short)
    z = torch.from_numpy(batch.z[:-1].copy()).cuda()
    z_before = z.clone()
    vt, cu_d, grid, text, cs, us = _device(batch)
    binding.rf_cfg_euler_step(z, vt, cu_d, grid, text, cs, us, 5.0, 0.25)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    assert torch.equal(z, z_before)
    # a consistent call afterwards succeeds and clears the flag
    got = _step(batch, 5.0, 0.25).cpu().numpy().astype(np.float64)
    check_close(got, _oracle(batch, 5.0, 0.25), "f32")
