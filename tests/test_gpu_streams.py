"""Calls on several streams that share the library's per-device workspace.

The forward, backward and projection each use one library-owned workspace
per device. A call enqueued on a stream other than the previous call's waits
on the device for that call, so interleaved calls on two streams give, bit
for bit, the outputs they give one at a time on one stream. The first call of
each pair is a long one (the 1024x1024 sample, 8 heads) so that, without that
wait, the second call's prologue would overwrite the workspace while the
first call's attention still reads it.
"""
import pytest
import torch

from text_image_diffusion_varlen_amd import binding, workloads

from gpu_common import device_inputs

pytestmark = pytest.mark.gpu


def _batch(w):
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    return q, k, v, cu, grid, text


def test_forward_on_two_streams_matches_one_stream():
    wa = workloads.make_custom([[64, 64]], [256], heads=8, head_dim=128, seed=3)
    wb = workloads.make_custom([[16, 40], [24, 24]], [77, 5], heads=8, head_dim=128, seed=4)
    a, b = _batch(wa), _batch(wb)
    ref_a = binding.attn_packed(*a)
    ref_b = binding.attn_packed(*b)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out_a, out_b = torch.empty_like(ref_a), torch.empty_like(ref_b)
    for rep in range(4):
        out_a.fill_(float("nan"))
        out_b.fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(2):
            with torch.cuda.stream(s1):
                binding.attn_packed(*a, out=out_a)
            with torch.cuda.stream(s2):
                binding.attn_packed(*b, out=out_b)
        torch.cuda.synchronize()
        assert binding.get_device_error() == binding.MF_OK
        assert torch.equal(out_a, ref_a), f"stream 1, repetition {rep}"
        assert torch.equal(out_b, ref_b), f"stream 2, repetition {rep}"


def test_backward_on_two_streams_matches_one_stream():
    wa = workloads.make_custom([[64, 64]], [256], heads=8, head_dim=128, seed=5)
    wb = workloads.make_custom([[20, 30], [8, 8]], [33, 0], heads=8, head_dim=128, seed=6)
    runs = []
    for w in (wa, wb):
        q, k, v, cu, grid, text = _batch(w)
        out, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
        dout = torch.randn(out.shape, generator=torch.Generator().manual_seed(w.tokens), dtype=torch.float32)
        dout = dout.to(torch.bfloat16).cuda()
        ref = binding.attn_packed_bwd(q, k, v, out, dout, lse, cu, grid, text)
        runs.append(((q, k, v, out, dout, lse, cu, grid, text), ref))
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    grads = [tuple(torch.empty_like(g) for g in ref) for _, ref in runs]
    for rep in range(3):
        for g in grads:
            for t in g:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        for (args, _), g, s in zip(runs, grads, (s1, s2)):
            with torch.cuda.stream(s):
                binding.attn_packed_bwd(*args, grads=g)
        torch.cuda.synchronize()
        assert binding.get_device_error() == binding.MF_OK
        for (_, ref), g in zip(runs, grads):
            for got, exp in zip(g, ref):
                assert torch.equal(got, exp), f"repetition {rep}"
