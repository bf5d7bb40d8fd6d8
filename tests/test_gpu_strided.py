"""The strided entry point (mf_attn_packed_strided, mf_tensor descriptors):
views of one fused [T][3][heads][d] projection buffer as q, k and v and a
head-major output view give exactly the bits of mf_attn_packed on contiguous
copies of the same values, and meet the oracle's bars; descriptors that would
let the output overlap itself or an input are refused; a metadata mismatch
writes nothing."""
import numpy as np
import pytest
import torch

from gpu_common import check_close, device_inputs, to_f64
from oracle import attention
from text_image_diffusion_varlen_amd import binding, workloads

pytestmark = pytest.mark.gpu


def _fused_views(q, k, v):
    T, H, D = q.shape
    buf = torch.stack([q, k, v], dim=1).contiguous()  # [T][3][H][D]
    return buf, buf[:, 0], buf[:, 1], buf[:, 2]


@pytest.mark.parametrize("config,heads", [("1024sq", 24), ("mixed", 8), ("tiny", 2)])
def test_strided_views_match_contiguous(config, heads):
    g, t = workloads.make_segments(config)
    base = workloads.make_workload(config)
    w = workloads.make_custom(g, t, heads=heads, head_dim=base.head_dim, dtype=base.dtype, seed=31,
                              scale=1.0 if base.dtype == "bf16" else 1.0 / 8.0, name=config)
    print(f"strided {config} T={w.tokens} H={heads} {w.dtype}", flush=True)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    ref = binding.attn_packed(q, k, v, cu, grid, text)
    buf, qs, ks, vs = _fused_views(q, k, v)
    assert qs.stride() == (3 * heads * w.head_dim, w.head_dim, 1)
    out_hm = torch.empty((heads, w.tokens, w.head_dim), dtype=q.dtype, device="cuda")
    out_view = out_hm.permute(1, 0, 2)  # [T][H][d] view of a head-major buffer
    binding.attn_packed_strided(qs, ks, vs, cu, grid, text, out_view)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    assert torch.equal(out_view, ref), "strided result differs from the contiguous call"
    # token-major output with a gap between heads (row pitch 2 d)
    wide = torch.zeros((w.tokens, heads, 2 * w.head_dim), dtype=q.dtype, device="cuda")
    binding.attn_packed_strided(qs, ks, vs, cu, grid, text, wide[:, :, : w.head_dim])
    torch.cuda.synchronize()
    assert torch.equal(wide[:, :, : w.head_dim], ref)
    assert torch.all(wide[:, :, w.head_dim:] == 0), "wrote outside the output view"
    sel = list(range(min(heads, 3)))
    exp = attention.joint_attention(w.q[:, sel], w.k[:, sel], w.v[:, sel], w.grid_hw, w.text_len)
    check_close(to_f64(out_view[:, sel]), exp, w.dtype)


def test_strided_rejects_bad_layouts():
    w = workloads.make_custom([[4, 4]], [3], heads=2, head_dim=128, dtype="bf16", seed=1)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    big = torch.zeros((w.tokens, 2, 256), dtype=torch.bfloat16, device="cuda")
    # heads of out overlapping (stride_head 64 < head_dim)
    over = big.view(-1)[: w.tokens * 256 * 2].as_strided((w.tokens, 2, 128), (512, 64, 1))
    with pytest.raises(binding.MFError) as e:
        binding.attn_packed_strided(q, k, v, cu, grid, text, over)
    assert e.value.code == binding.MF_ERR_INVALID_ARG
    # out overlapping an input
    buf, qs, ks, vs = _fused_views(q, k, v)
    with pytest.raises(binding.MFError) as e:
        binding.attn_packed_strided(qs, ks, vs, cu, grid, text, buf[:, 2])
    assert e.value.code == binding.MF_ERR_INVALID_ARG
    # stride not a multiple of 16 bytes
    odd = torch.zeros((w.tokens, 2, 131), dtype=torch.bfloat16, device="cuda")[:, :, :128]
    with pytest.raises(binding.MFError) as e:
        binding.attn_packed_strided(q, k, v, cu, grid, text, odd)
    assert e.value.code == binding.MF_ERR_INVALID_ARG


def test_strided_metadata_mismatch_writes_nothing():
    w = workloads.make_custom([[4, 4], [3, 5]], [2, 1], heads=2, head_dim=128, dtype="bf16", seed=2)
    q, k, v, grid, text = device_inputs(w)
    _, qs, ks, vs = _fused_views(q, k, v)
    bad_cu = torch.tensor([0, 17, w.tokens], dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 3.0)
    binding.attn_packed_strided(qs, ks, vs, bad_cu, grid, text, out)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    assert torch.all(out == 3.0)
    # reported once: a later check with no failing call in between is clean
    assert binding.get_device_error() == binding.MF_OK
