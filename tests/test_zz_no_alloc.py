"""The allocation-free forward (mf_attn_packed_noalloc) against the allocating
entry point (mf_attn_packed) and the fp64 oracle.

Both calls run the same kernels; the allocation-free one keeps its workspace
in a fixed static device array and never splits a last round, so on batches
that mf_attn_packed does not split either the two outputs must agree bit for
bit, and both must meet the parity bars against the oracle. Two calls in a
row (a large batch, then a smaller one) check that the scratch left behind by
the first call does not leak into the second; a call that does not fit the
fixed size is refused; a metadata mismatch writes nothing and is reported by
mf_get_device_error; the call can be captured into a HIP graph after one
eager call and replayed.
"""
import numpy as np
import pytest
import torch

from gpu_common import check_close, device_inputs, to_f64
from oracle import attention
from text_image_diffusion_varlen_amd import binding, workloads

pytestmark = pytest.mark.gpu


def _both(w):
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    ref = binding.attn_packed(q, k, v, cu, grid, text)
    got = binding.attn_packed_noalloc(q, k, v, cu, grid, text, out=torch.empty_like(q))
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    return got, ref


def test_noalloc_matches_allocating_entry_point_large_then_small():
    big = workloads.make_workload("1024sq")
    small = workloads.make_custom([[6, 11], [3, 3], [1, 40], [9, 2]], [20, 0, 5, 77], heads=4, head_dim=128,
                                  dtype="bf16", seed=41, name="small")
    sel = [0, 8, 23]
    for w in (big, small):
        print(f"noalloc {w.name} T={w.tokens} H={w.heads}", flush=True)
        got, ref = _both(w)
        assert torch.equal(got, ref), f"{w.name}: allocation-free output differs from mf_attn_packed"
        heads = sel if w.heads > 4 else list(range(w.heads))
        exp = attention.joint_attention(w.q[:, heads], w.k[:, heads], w.v[:, heads], w.grid_hw, w.text_len)
        check_close(to_f64(got[:, heads]), exp, "bf16")


@pytest.mark.parametrize("config", ["tiny", "mixed"])
def test_noalloc_configs(config):
    w = workloads.make_workload(config)
    print(f"noalloc {config} T={w.tokens} H={w.heads} {w.dtype}", flush=True)
    got, ref = _both(w)
    assert torch.equal(got, ref)
    if w.heads <= 2:
        check_close(to_f64(got), attention.joint_attention(w.q, w.k, w.v, w.grid_hw, w.text_len), w.dtype)


def test_noalloc_rejects_batches_beyond_the_scratch():
    T = 40000  # 24 heads x 128 bf16: about 480 MB of key / value buffers
    q = torch.zeros((T, 24, 128), dtype=torch.bfloat16, device="cuda")
    grid = torch.tensor([[100, 398]], dtype=torch.int32, device="cuda")
    text = torch.tensor([T - 100 * 398], dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(binding.MFError) as e:
        binding.attn_packed_noalloc(q, q, q, cu, grid, text, out=torch.empty_like(q))
    assert e.value.code == binding.MF_ERR_UNSUPPORTED
    assert "maximum" in str(e.value)


def test_noalloc_metadata_mismatch_writes_nothing():
    w = workloads.make_custom([[4, 4], [3, 5]], [2, 1], heads=2, head_dim=128, dtype="bf16", seed=2)
    q, k, v, grid, text = device_inputs(w)
    bad_cu = torch.tensor([0, 17, w.tokens], dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 3.0)
    binding.attn_packed_noalloc(q, k, v, bad_cu, grid, text, out=out)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    assert torch.all(out == 3.0)
    got, ref = _both(w)  # a consistent call afterwards succeeds and clears the flag
    assert torch.equal(got, ref)


def test_noalloc_graph_replays():
    """Captured after one eager call (the one-time setup), replayed with new
    input values and eager calls on other batches in between; every replay
    equals an eager call on the same inputs bit for bit."""
    w = workloads.make_workload("mixed", seed=21)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    out = torch.empty_like(q)
    binding.attn_packed_noalloc(q, k, v, cu, grid, text, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.attn_packed_noalloc(q, k, v, cu, grid, text, out=out)
    other = workloads.make_custom([[7, 9], [2, 30]], [12, 3], heads=24, head_dim=128, dtype="bf16", seed=5)
    rng = np.random.default_rng(3)
    for rep in range(3):
        for t in (q, k, v):
            t.copy_(torch.from_numpy(rng.standard_normal(t.shape, dtype=np.float32)).to(t.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        _both(other)  # other work on the same scratch between replays
        eager = binding.attn_packed(q, k, v, cu, grid, text)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep} differs from an eager call"
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
