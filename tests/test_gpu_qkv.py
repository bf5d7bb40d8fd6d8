"""GPU parity of the modality-specific RMSNorm + packed QKV projection
(mf_qkv_fold_weights, mf_qkv_rmsnorm) against the fp64 oracle.

Outputs are ~N(0, 1) bf16 values, so the bf16 bar of the attention applies:
max abs <= 2e-2, mean abs <= 2e-3. The folded weights are compared bit for bit
with bf16(gamma * W) formed in float32 on the host and put in the tiled order
the header documents.
"""
import numpy as np
import pytest
import torch

from oracle import packing, projection
from text_image_diffusion_varlen_amd import binding, workloads

from gpu_common import check_close, to_f64

pytestmark = pytest.mark.gpu


def _run(grid, text, hidden, heads, d, frames=None, seed=0):
    x, wt, wi, gt, gi = workloads.make_qkv_inputs(grid, text, hidden, heads, d, frames, seed)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()  # noqa: E731
    wf = binding.qkv_fold_weights(bf(wt), bf(wi), torch.from_numpy(gt).cuda(), torch.from_numpy(gi).cuda(), heads, d)
    cu = torch.from_numpy(packing.cu_seqlens(grid, text, frames)).cuda()
    grid_d = torch.tensor(np.asarray(grid, np.int32).reshape(-1, 2), device="cuda")
    text_d = torch.tensor(np.asarray(text, np.int32), device="cuda")
    fr = None if frames is None else torch.tensor(np.asarray(frames, np.int32), device="cuda")
    q, k, v = binding.qkv_rmsnorm(bf(x), wf, cu, grid_d, text_d, heads, d, frames=fr)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    return (x, wt, wi, gt, gi), wf, (q, k, v)


def _check(grid, text, hidden, heads, d, frames=None, seed=0):
    print(f"qkv grid={np.asarray(grid).tolist()[:4]} hidden={hidden} hd={heads * d}", flush=True)
    (x, wt, wi, gt, gi), wf, got = _run(grid, text, hidden, heads, d, frames, seed)
    exp = projection.rmsnorm_qkv(x, wt, wi, gt, gi, grid, text, heads, d, frames)
    for g, e in zip(got, exp):
        check_close(to_f64(g), e, "bf16")
    return wf, (wt, wi, gt, gi)


def _tiled(a):
    """Chunk order of the projection's tiled weights: stacked row R, 8-channel chunk
    g -> 16-byte chunk ((R // 256) * (C // 64) + g // 8) * 2048 + (g % 8) * 256 + R % 256."""
    R, C = a.shape
    chunks = a.reshape(R, C // 8, 8)
    out = np.empty_like(chunks.reshape(-1, 8))
    r = np.arange(R)[:, None]
    g = np.arange(C // 8)[None, :]
    idx = ((r // 256) * (C // 64) + g // 8) * 2048 + (g % 8) * 256 + r % 256
    out[idx.reshape(-1)] = chunks.reshape(-1, 8)
    return out.reshape(-1)


def test_fold_weights_bitwise():
    wf, (wt, wi, gt, gi) = _check([[3, 5]], [7], 128, 2, 128, seed=1)
    ref = np.concatenate([workloads.f32_to_bf16_bits((w * g[None, :]).astype(np.float32))
                          for w, g in ((wt, gt), (wi, gi))])
    got = wf.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    assert np.array_equal(got, _tiled(ref))


@pytest.mark.parametrize("grid,text,frames", [
    ([[64, 64]], [256], None),                                   # the 1024^2 sample
    ([[32, 128], [128, 32], [48, 84]], [77, 200, 256], None),    # mixed aspect ratios
    ([[1, 1], [2, 3], [1, 7], [5, 1]], [0, 0, 3, 0], None),      # tiny grids, mostly no prompt
    ([[16, 16]], [0], None),                                     # no text token at all
    ([[4, 4], [2, 8]], [10, 1], [2, 3]),                         # editing samples (frames)
])
def test_qkv_parity(grid, text, frames):
    _check(grid, text, 3072 if grid == [[64, 64]] else 512, 4 if grid == [[64, 64]] else 2, 128, frames, seed=2)


def test_qkv_24_heads_full_width():
    """The 4B model's attention width: 24 heads x 128 from hidden 3072, on a
    batch whose text and visual row counts are not multiples of the tile."""
    _check([[20, 30], [9, 13]], [100, 33], 3072, 24, 128, seed=3)


def test_qkv_head_dim_64_and_many_samples():
    rng = np.random.default_rng(4)
    grid = rng.integers(1, 9, size=(300, 2)).tolist()
    text = rng.integers(0, 12, size=300).tolist()
    _check(grid, text, 256, 4, 64, seed=4)


def test_qkv_metadata_mismatch_writes_nothing():
    grid, text, hidden, heads, d = [[4, 4], [3, 5]], [2, 1], 128, 2, 128
    x, wt, wi, gt, gi = workloads.make_qkv_inputs(grid, text, hidden, heads, d, seed=5)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()  # noqa: E731
    wf = binding.qkv_fold_weights(bf(wt), bf(wi), torch.from_numpy(gt).cuda(), torch.from_numpy(gi).cuda(), heads, d)
    grid_d = torch.tensor(grid, dtype=torch.int32, device="cuda")
    text_d = torch.tensor(text, dtype=torch.int32, device="cuda")
    bad_cu = torch.tensor([0, 17, 34], dtype=torch.int32, device="cuda")
    out = tuple(torch.full((34, heads, d), 5.0, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    binding.qkv_rmsnorm(bf(x), wf, bad_cu, grid_d, text_d, heads, d, out=out)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    for t in out:
        assert torch.all(t == 5.0)
    _check(grid, text, hidden, heads, d, seed=5)  # a consistent call clears the flag


def test_qkv_rejects_unsupported_shapes():
    x = torch.zeros((10, 96), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((2, 3 * 256, 96), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 10], dtype=torch.int32, device="cuda")
    g = torch.tensor([[3, 3]], dtype=torch.int32, device="cuda")
    t = torch.tensor([1], dtype=torch.int32, device="cuda")
    with pytest.raises(binding.MFError) as e:
        binding.qkv_rmsnorm(x, w, cu, g, t, 2, 128)
    assert e.value.code == binding.MF_ERR_UNSUPPORTED


def test_halved_last_round_matches_whole_units(tmp_path):
    """The 1024^2 sample at 24 x 128 (hidden 3072) has 612 GEMM units; on a
    256-CU device the last 100 run as 128-feature halves. A child process with
    MF_ATTN_SPLIT=0 runs every unit whole; q, k, v must agree bit for bit
    (each output element is summed in the same order either way)."""
    import os
    import subprocess
    import sys

    args = ([[64, 64]], [256], 3072, 24, 128)
    _, _, got = _run(*args, seed=6)
    here = os.path.dirname(os.path.abspath(__file__))
    out = tmp_path / "whole.pt"
    child = (
        "import sys, torch\n"
        f"sys.path[:0] = [{here!r}, {os.path.dirname(here)!r}]\n"
        "import test_gpu_qkv as t\n"
        f"_, _, o = t._run(*{args!r}, seed=6)\n"
        f"torch.save([x.cpu() for x in o], {str(out)!r})\n"
    )
    print("qkv halved vs whole: child process with MF_ATTN_SPLIT=0", flush=True)
    subprocess.run([sys.executable, "-c", child], env=dict(os.environ, MF_ATTN_SPLIT="0"), check=True, timeout=300)
    ref = torch.load(out, weights_only=True)
    for name, a, b in zip("qkv", got, ref):
        assert torch.equal(a.cpu(), b), f"{name} differs between halved and whole units"
