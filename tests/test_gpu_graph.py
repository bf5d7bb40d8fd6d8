"""HIP-graph capture of the stream-ordered entry points.

The packed forward, the packed backward, the guided Euler step, the
RMSNorm + QKV projection prologue, and a forward + backward whose kernels all
split their last round, are each captured once (after an eager call
has sized the library's workspaces and uploaded its RoPE table), then replayed
several times with new values written into the captured input buffers, with
eager library calls, other device work and host synchronizations between the
replays. Every replay must equal an
eager call on the same inputs bit for bit (all kernels are deterministic).
"""
import pytest
import torch

from gpu_common import device_inputs
from text_image_diffusion_varlen_amd import binding, workloads

pytestmark = pytest.mark.gpu


def _mixed():
    w = workloads.make_workload("mixed")
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    return w, q, k, v, grid, text, cu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _new_inputs(dst, src, rep):
    """Writes a different but valid input into each captured buffer."""
    for d, s in zip(dst, src):
        d.copy_(s.roll(97 * (rep + 1), dims=0) * (1.0 + 0.125 * rep))


def test_forward_graph_replays_match_eager():
    w, q, k, v, grid, text, cu = _mixed()
    print(f"graph forward mixed T={w.tokens}", flush=True)
    out_e, out_g = torch.empty_like(q), torch.empty_like(q)
    binding.attn_packed(q, k, v, cu, grid, text, out=out_e)  # sizes the workspace
    torch.cuda.synchronize()
    qg, kg, vg = q.clone(), k.clone(), v.clone()
    g = _capture(lambda: binding.attn_packed(qg, kg, vg, cu, grid, text, out=out_g))
    for rep in range(4):
        _new_inputs((qg, kg, vg), (q, k, v), rep)
        g.replay()
        torch.cuda.synchronize()
        binding.attn_packed(qg, kg, vg, cu, grid, text, out=out_e)
        assert torch.isfinite((out_e.float() * 2).sum())  # other device work between replays
        torch.cuda.synchronize()
        assert binding.get_device_error() == binding.MF_OK, binding.last_error()
        assert torch.equal(out_g, out_e), f"replay {rep} differs from the eager call"


def test_backward_graph_replays_match_eager():
    w, q, k, v, grid, text, cu = _mixed()
    print(f"graph backward mixed T={w.tokens}", flush=True)
    out, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
    d_out = torch.randn(q.shape, generator=torch.Generator(device="cuda").manual_seed(11), device="cuda",
                        dtype=torch.float32).to(q.dtype)
    grads_e = tuple(torch.empty_like(q) for _ in range(3))
    grads_g = tuple(torch.empty_like(q) for _ in range(3))
    binding.attn_packed_bwd(q, k, v, out, d_out, lse, cu, grid, text, grads=grads_e)  # sizes the workspace
    torch.cuda.synchronize()
    dog = d_out.clone()
    g = _capture(lambda: binding.attn_packed_bwd(q, k, v, out, dog, lse, cu, grid, text, grads=grads_g))
    for rep in range(3):
        _new_inputs((dog,), (d_out,), rep)
        g.replay()
        torch.cuda.synchronize()
        binding.attn_packed_bwd(q, k, v, out, dog, lse, cu, grid, text, grads=grads_e)
        torch.cuda.synchronize()
        assert binding.get_device_error() == binding.MF_OK, binding.last_error()
        for name, a, b in zip(("dq", "dk", "dv"), grads_g, grads_e):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_cfg_step_graph_replays_match_eager():
    b = workloads.make_cfg_batch([(16, 24), (32, 8), (12, 12)], channels=64, seed=6)
    print(f"graph cfg step images={len(b.cond_seg)}", flush=True)
    grid = torch.from_numpy(b.grid_hw).cuda()
    text = torch.from_numpy(b.text_len).cuda()
    cu, _, _ = binding.build_metadata(grid, text, b.tokens)
    cs = torch.from_numpy(b.cond_seg).cuda()
    us = torch.from_numpy(b.uncond_seg).cuda()
    z0 = torch.from_numpy(b.z).cuda()
    v = torch.from_numpy(b.v).to(torch.bfloat16).cuda()
    z_e, z_g = z0.clone(), z0.clone()
    step = lambda z: binding.rf_cfg_euler_step(z, v, cu, grid, text, cs, us, 5.0, 0.25)  # noqa: E731
    step(torch.empty_like(z0).copy_(z0))  # first call on the device outside the capture
    torch.cuda.synchronize()
    g = _capture(lambda: step(z_g))
    z_g.copy_(z0)  # the capture did not run the step
    for rep in range(4):
        g.replay()
        step(z_e)
        torch.cuda.synchronize()
        assert binding.get_device_error() == binding.MF_OK, binding.last_error()
        assert torch.equal(z_g, z_e), f"replay {rep} differs from the eager step"


def test_qkv_prologue_graph_replays_match_eager():
    grid_hw = [(16, 24), (8, 40), (20, 20)]
    text_len = [77, 130, 0]
    heads, d = 4, 64
    hidden = heads * d
    x, wt, wi, gt, gi = workloads.make_qkv_inputs(grid_hw, text_len, hidden, heads, d, seed=4)
    print(f"graph qkv prologue T={x.shape[0]}", flush=True)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()  # noqa: E731
    grid = torch.tensor(grid_hw, dtype=torch.int32).cuda()
    text = torch.tensor(text_len, dtype=torch.int32).cuda()
    cu, _, _ = binding.build_metadata(grid, text, x.shape[0])
    wf = binding.qkv_fold_weights(bf(wt), bf(wi), torch.from_numpy(gt).cuda(), torch.from_numpy(gi).cuda(), heads, d)
    x0 = bf(x)
    T = x0.shape[0]
    out_e = tuple(torch.empty((T, heads, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    out_g = tuple(torch.empty((T, heads, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    binding.qkv_rmsnorm(x0, wf, cu, grid, text, heads, d, out=out_e)  # sizes the workspace
    torch.cuda.synchronize()
    xg = x0.clone()
    g = _capture(lambda: binding.qkv_rmsnorm(xg, wf, cu, grid, text, heads, d, out=out_g))
    for rep in range(3):
        _new_inputs((xg,), (x0,), rep)
        g.replay()
        torch.cuda.synchronize()
        binding.qkv_rmsnorm(xg, wf, cu, grid, text, heads, d, out=out_e)
        torch.cuda.synchronize()
        assert binding.get_device_error() == binding.MF_OK, binding.last_error()
        for name, a, b in zip("qkv", out_g, out_e):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_split_paths_graph_replays_match_eager():
    """A 9000-token sample with 2 heads: the forward, dK/dV and dQ kernels all
    split their last round (pieces, partial slots, merges). The forward with
    LSE and the backward are captured together and replayed against eager calls."""
    w = workloads.make_custom([[88, 100]], [200], heads=2, head_dim=128, dtype="bf16", seed=19, name="split_graph")
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    print(f"graph split paths T={w.tokens}", flush=True)
    d_out = torch.randn(q.shape, generator=torch.Generator(device="cuda").manual_seed(12), device="cuda",
                        dtype=torch.float32).to(q.dtype)
    lse_e, lse_g = (torch.empty((w.heads, w.tokens), dtype=torch.float32, device="cuda") for _ in range(2))
    out_e, out_g = torch.empty_like(q), torch.empty_like(q)
    grads_e = tuple(torch.empty_like(q) for _ in range(3))
    grads_g = tuple(torch.empty_like(q) for _ in range(3))

    def step(qq, out, lse, grads):
        binding.attn_packed_lse(qq, k, v, cu, grid, text, out=out, lse=lse)
        binding.attn_packed_bwd(qq, k, v, out, d_out, lse, cu, grid, text, grads=grads)

    step(q, out_e, lse_e, grads_e)  # sizes both workspaces
    torch.cuda.synchronize()
    qg = q.clone()
    g = _capture(lambda: step(qg, out_g, lse_g, grads_g))
    for rep in range(3):
        _new_inputs((qg,), (q,), rep)
        g.replay()
        torch.cuda.synchronize()
        step(qg, out_e, lse_e, grads_e)
        torch.cuda.synchronize()
        assert binding.get_device_error() == binding.MF_OK, binding.last_error()
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e), f"replay {rep}: forward differs"
        for name, a, b in zip(("dq", "dk", "dv"), grads_g, grads_e):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
