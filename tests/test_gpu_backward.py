"""GPU parity of the packed backward (mf_attn_packed_lse + mf_attn_packed_bwd)
against the fp64 oracle (joint_attention_lse, joint_attention_backward).

Bars. Gradients shrink like 1/sqrt(L), so they are compared relative to their
own scale: max |got - ref| <= 2e-2 * max |ref| + 1e-5 and mean |got - ref| <=
1e-2 * mean |ref| + 1e-5, per gradient (the 1e-5 floor covers gradients that
vanish exactly, e.g. dq and dk of a one-token sample, where fp32 rounding of
dP - D leaves ~1e-7). The kernel rounds P and dX to bf16 (relative error
2^-9 each) as MFMA operands and the gradients themselves to bf16, and reads
the forward's bf16 output in D = rowsum(dO * O); those roundings stay well
inside 1% of the gradient's scale. LSE: the forward normalizes by the row sum
of the bf16-rounded P it multiplies into V (so that O is exactly that
weighted mean), and bf16's unit roundoff is 2^-8, so the stored LSE can
differ from the exact one by up to ln(1 + 2^-8) = 3.9e-3; the bf16 rounding of
the rotated operands adds a score shift that long rows average away but rows
of a few keys do not (the per-row bar of gpu_common.check_lse).
"""
import numpy as np
import pytest
import torch

from oracle import attention
from text_image_diffusion_varlen_amd import binding, workloads

from gpu_common import check_lse, device_inputs, to_f64

pytestmark = pytest.mark.gpu
GRAD_TOL = (2e-2, 1e-2)  # (max, mean) relative to the reference's own max / mean magnitude
GRAD_FLOOR = 1e-5


def _d_out(w, seed=9):
    rng = np.random.default_rng(seed)
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(rng.standard_normal(w.q.shape, dtype=np.float32)))


def _run(w, do):
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    out, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
    dot = torch.from_numpy(do).to(torch.bfloat16).cuda()
    dq, dk, dv = binding.attn_packed_bwd(q, k, v, out, dot, lse, cu, grid, text)
    torch.cuda.synchronize()
    assert binding.get_device_error() == binding.MF_OK, binding.last_error()
    return out, lse, dq, dk, dv


def _check_grad(name, got, ref):
    err = np.abs(got - ref)
    scale_max, scale_mean = np.abs(ref).max(), np.abs(ref).mean()
    assert np.isfinite(got).all(), f"{name}: non-finite"
    print(f"  {name}: max err {err.max():.3e} (ref max {scale_max:.3e}), mean err {err.mean():.3e} "
          f"(ref mean {scale_mean:.3e})")
    assert err.max() <= GRAD_TOL[0] * scale_max + GRAD_FLOOR, name
    assert err.mean() <= GRAD_TOL[1] * scale_mean + GRAD_FLOOR, name


def _full_check(w):
    print(f"backward {w.name} T={w.tokens} n={w.n_seg} H={w.heads} d={w.head_dim}", flush=True)
    do = _d_out(w)
    out, lse, dq, dk, dv = _run(w, do)
    ref_lse = attention.joint_attention_lse(w.q, w.k, w.grid_hw, w.text_len)
    lerr = check_lse(lse.cpu().numpy(), ref_lse, w)
    print(f"  lse: max err {lerr:.3e}")
    rq, rk, rv = attention.joint_attention_backward(w.q, w.k, w.v, do, w.grid_hw, w.text_len)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check_grad(name, to_f64(g), r)


EDGE = {
    "one_token": ([[1, 1]], [0]),
    "thin": ([[1, 5], [5, 1], [1, 1]], [0, 3, 7]),
    "tile_edges": ([[8, 8], [1, 63], [2, 32], [1, 127], [1, 128], [3, 43]], [0, 1, 1, 0, 1, 0]),
    "many": (np.random.default_rng(31).integers(1, 12, size=(40, 2)).tolist(),
             np.random.default_rng(32).integers(0, 20, size=40).tolist()),
    "long_prompt": ([[2, 2]], [300]),
    "key_blocks": ([[9, 29], [16, 16], [1, 200]], [20, 0, 57]),  # 281, 256, 257 tokens: 128-key block edges
    "max_samples": (np.random.default_rng(33).integers(1, 4, size=(4096, 2)).tolist(),  # 4096 samples
                    np.random.default_rng(34).integers(0, 4, size=4096).tolist()),
}


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("d", [64, 128])
def test_backward_edge_cases(name, d):
    grid, text = EDGE[name]
    _full_check(workloads.make_custom(grid, text, heads=3, head_dim=d, dtype="bf16", seed=11, name=name))


@pytest.mark.parametrize("config", ["1024sq", "mixed"])
def test_backward_configs_two_heads(config):
    """The 1024^2 and mixed batches at their real lengths, two heads (the oracle's
    fp64 backward over all 24 heads takes minutes)."""
    g, t = workloads.make_segments(config)
    _full_check(workloads.make_custom(g, t, heads=2, head_dim=128, dtype="bf16", seed=12, name=config))


def _head_subset(w, heads):
    return workloads.Workload(f"{w.name}[heads {heads}]", w.grid_hw, w.text_len, len(heads), w.head_dim, w.dtype,
                              w.q[:, heads], w.k[:, heads], w.v[:, heads], seed=w.seed)


# (config, heads, compared heads): the real head counts run the XCD-aware dQ
# order (heads a multiple of 8, at least 16) and, on 1024sq with 24 heads, the
# dK/dV split plan (816 units on 256 CUs, the last 48 cut into 4 query ranges).
ALL_HEADS = {
    "1024sq_h24": ("1024sq", 24, [0, 7, 8, 23]),
    "mixed_h24": ("mixed", 24, [0, 9, 16, 23]),
    "1024sq_h16": ("1024sq", 16, [0, 9, 15]),
}


@pytest.mark.parametrize("name", sorted(ALL_HEADS))
def test_backward_configs_all_heads(name):
    """The 1024^2 and mixed batches at their real head count on the GPU; heads
    are independent, so a few heads are compared with the oracle run on those
    head slices alone (LSE, dq, dk, dv, every element of those heads)."""
    config, heads, sel = ALL_HEADS[name]
    g, t = workloads.make_segments(config)
    w = workloads.make_custom(g, t, heads=heads, head_dim=128, dtype="bf16", seed=14, name=config)
    print(f"backward {name} T={w.tokens} n={w.n_seg} H={heads} compared heads {sel}", flush=True)
    do = _d_out(w)
    out, lse, dq, dk, dv = _run(w, do)
    ws = _head_subset(w, sel)
    dos = do[:, sel]
    lerr = check_lse(lse.cpu().numpy()[sel], attention.joint_attention_lse(ws.q, ws.k, ws.grid_hw, ws.text_len), ws)
    print(f"  lse: max err {lerr:.3e}")
    rq, rk, rv = attention.joint_attention_backward(ws.q, ws.k, ws.v, dos, ws.grid_hw, ws.text_len)
    for gname, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check_grad(gname, to_f64(g[:, sel]), r)
    for gname, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(g.float()).all(), f"{gname}: non-finite"


def test_forward_with_lse_matches_forward_bitwise():
    w = workloads.make_workload("mixed", seed=24)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    a = binding.attn_packed(q, k, v, cu, grid, text)
    b, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.isfinite(lse).all()


def test_backward_deterministic_and_sample_independent():
    """No atomics: two runs agree bit for bit, and each sample's gradients are
    the same bits when it is run alone."""
    w = workloads.make_custom([[5, 7], [12, 3], [1, 1], [8, 16]], [9, 0, 4, 77], heads=2, head_dim=128,
                              dtype="bf16", seed=13)
    do = _d_out(w)
    r1 = _run(w, do)
    r2 = _run(w, do)
    for x, y in zip(r1[2:], r2[2:]):
        assert torch.equal(x, y)
    cu = np.concatenate([[0], np.cumsum(w.text_len + w.grid_hw[:, 0] * w.grid_hw[:, 1])])
    for i in range(w.n_seg):
        a, b = int(cu[i]), int(cu[i + 1])
        wi = workloads.Workload("one", w.grid_hw[i:i + 1], w.text_len[i:i + 1], w.heads, w.head_dim, w.dtype,
                                w.q[a:b], w.k[a:b], w.v[a:b])
        ri = _run(wi, do[a:b])
        for x, y in zip(ri[2:], r1[2:]):
            assert torch.equal(x, y[a:b]), f"sample {i}"


def test_backward_metadata_mismatch_writes_nothing():
    w = workloads.make_custom([[4, 4], [3, 5]], [2, 1], heads=2, head_dim=128, dtype="bf16", seed=2)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    out, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
    dot = torch.from_numpy(_d_out(w)).to(torch.bfloat16).cuda()
    bad_cu = torch.tensor([0, 17, w.tokens], dtype=torch.int32, device="cuda")
    grads = tuple(torch.full_like(q, 3.0) for _ in range(3))
    binding.attn_packed_bwd(q, k, v, out, dot, lse, bad_cu, grid, text, grads=grads)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    for g in grads:
        assert torch.all(g == 3.0)
    _run(w, _d_out(w))  # a consistent call afterwards succeeds and clears the flag


def test_backward_rejects_f32():
    w = workloads.make_custom([[2, 2]], [1], heads=1, head_dim=64, dtype="f32", seed=1)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    out, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
    with pytest.raises(binding.MFError) as e:
        binding.attn_packed_bwd(q, k, v, out, torch.zeros_like(q), lse, cu, grid, text)
    assert e.value.code == binding.MF_ERR_UNSUPPORTED
