"""GPU parity of the packed joint attention path against the fp64 oracle.

Tolerances (fp64 oracle on the same bf16/f32 inputs): bf16 max abs <= 2e-2 and
mean abs <= 2e-3; f32 max abs <= 1e-5. Small and medium workloads are compared
element by element over the whole output; the 2048x2048 and training-style
workloads on seeded samples of output rows (first/last rows of every sample,
prompt rows, and random rows), since the oracle evaluates those row by row.
"""
import numpy as np
import pytest
import torch

from oracle import attention
from text_image_diffusion_varlen_amd import binding, workloads

from gpu_common import check_close, device_inputs, run_attention, to_f64

pytestmark = pytest.mark.gpu


def _full_check(w):
    print(f"attention {w.name} T={w.tokens} n={w.n_seg}", flush=True)
    got = to_f64(run_attention(w))
    exp = attention.joint_attention(w.q, w.k, w.v, w.grid_hw, w.text_len)
    return check_close(got, exp, w.dtype)


@pytest.mark.parametrize("config", ["tiny", "1024sq", "mixed"])
def test_attention_configs_full(config):
    _full_check(workloads.make_workload(config))


def _sample_rows(w, n_random, seed):
    cu = np.concatenate([[0], np.cumsum(w.text_len.astype(np.int64) + w.grid_hw[:, 0] * w.grid_hw[:, 1])])
    rows = set()
    for i in range(w.n_seg):
        a, b = int(cu[i]), int(cu[i + 1])
        rows.update([a, b - 1, min(a + int(w.text_len[i]), b - 1)])
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, w.tokens, size=n_random).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("config", ["2048sq", "train65k"])
def test_attention_configs_sampled(config):
    w = workloads.make_workload(config)
    print(f"attention {config} T={w.tokens} n={w.n_seg}", flush=True)
    got = run_attention(w)
    rows = _sample_rows(w, 384, seed=5)
    g = to_f64(got[torch.from_numpy(rows).cuda()])
    exp = attention.joint_attention_rows(w.q, w.k, w.v, w.grid_hw, w.text_len, rows)
    check_close(g, exp, w.dtype)
    # every output row finite
    assert torch.isfinite(got.float()).all()


@pytest.mark.parametrize("seed", [20, 21, 22, 23, 24])
def test_attention_mixed_seeds(seed):
    _full_check(workloads.make_workload("mixed", seed=seed))


EDGE = {
    # single token: output is v
    "one_token": ([[1, 1]], [0]),
    # image-only and prompt-heavy samples, grids one row or one column wide
    "thin": ([[1, 5], [5, 1], [1, 1]], [0, 3, 7]),
    # lengths around the 64-key and 128-query tile edges
    "tile_edges": ([[8, 8], [1, 63], [2, 32], [1, 127], [1, 128], [3, 43]], [0, 1, 1, 0, 1, 0]),
    # many small samples
    "many": (np.random.default_rng(31).integers(1, 12, size=(40, 2)).tolist(),
             np.random.default_rng(32).integers(0, 20, size=40).tolist()),
    # long prompt, tiny image
    "long_prompt": ([[2, 2]], [300]),
    # the maximum number of samples (4096), each a few tokens: one query tile and
    # one key tile per sample, 4096 tile-table entries
    "max_samples": (np.random.default_rng(33).integers(1, 4, size=(4096, 2)).tolist(),
                    np.random.default_rng(34).integers(0, 4, size=4096).tolist()),
}


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_attention_edge_cases(name, dtype, d):
    grid, text = EDGE[name]
    scale = 1.0 if dtype == "bf16" else 0.125
    w = workloads.make_custom(grid, text, heads=3, head_dim=d, dtype=dtype, seed=9, scale=scale, name=name)
    _full_check(w)


@pytest.mark.parametrize("heads", [1, 7, 40])
@pytest.mark.parametrize("d", [64, 128])
def test_attention_head_counts(heads, d):
    """Head counts that are not multiples of the XCD count, one head and many:
    the workgroup id splits into (tile, head) differently for each."""
    w = workloads.make_custom([[9, 14], [1, 70], [12, 12]], [40, 0, 77], heads=heads, head_dim=d, dtype="bf16",
                              seed=heads + d, name=f"heads{heads}")
    _full_check(w)


def test_attention_largest_grid_sampled():
    """The largest supported sample: a 512 x 512 grid (positions up to 511 on
    both axes, 4100 key tiles) after a 256-token prompt, plus a small sample
    after it; checked on seeded rows including the grid's corners."""
    w = workloads.make_custom([[512, 512], [3, 4]], [256, 5], heads=2, head_dim=128, dtype="bf16", seed=12,
                              name="grid512")
    print(f"attention grid512 T={w.tokens}", flush=True)
    got = run_attention(w)
    t0 = 256  # first image token of the big sample
    corners = [t0, t0 + 511, t0 + 511 * 512, t0 + 512 * 512 - 1]
    rows = np.unique(np.concatenate([_sample_rows(w, 96, seed=13), corners]))
    g = to_f64(got[torch.from_numpy(rows).cuda()])
    exp = attention.joint_attention_rows(w.q, w.k, w.v, w.grid_hw, w.text_len, rows)
    check_close(g, exp, w.dtype)
    assert torch.isfinite(got.float()).all()


def test_one_token_returns_v():
    w = workloads.make_custom([[1, 1], [1, 1]], [0, 0], heads=2, head_dim=128, dtype="bf16", seed=1)
    got = run_attention(w)
    assert torch.equal(got.float().cpu(), torch.from_numpy(w.v))


def test_packed_equals_each_sample_alone_bitwise():
    """Query tiles are sample-relative, so a sample's output bits do not depend on
    what else is packed with it, as long as neither call splits its last round
    (batches whose mean sample length is below the split threshold, like this
    one, never split; a split sums the split units' keys in pieces)."""
    w = workloads.make_workload("mixed", seed=20)
    packed = run_attention(w)
    cu = np.concatenate([[0], np.cumsum(w.text_len + w.grid_hw[:, 0] * w.grid_hw[:, 1])])
    for i in range(w.n_seg):
        a, b = int(cu[i]), int(cu[i + 1])
        wi = workloads.Workload("one", w.grid_hw[i : i + 1], w.text_len[i : i + 1], w.heads, w.head_dim,
                                w.dtype, w.q[a:b], w.k[a:b], w.v[a:b])
        alone = run_attention(wi)
        assert torch.equal(alone, packed[a:b]), f"sample {i} differs"


def test_no_leakage_between_samples_bitwise():
    """Scale every other sample's keys and values by 256: any attention weight
    that crossed a sample boundary would move this sample's output. Tiles are
    sample-relative, so the sample's output bits must not change at all."""
    w = workloads.make_workload("mixed", seed=23)
    base = run_attention(w)
    cu = np.concatenate([[0], np.cumsum(w.text_len + w.grid_hw[:, 0] * w.grid_hw[:, 1])])
    i = 2
    a, b = int(cu[i]), int(cu[i + 1])
    k2, v2 = w.k.copy(), w.v.copy()
    big = np.float32(256.0)  # exact in bf16
    for arr in (k2, v2):
        arr[:a] *= big
        arr[b:] *= big
    wl = workloads.Workload("loud", w.grid_hw, w.text_len, w.heads, w.head_dim, w.dtype, w.q, k2, v2)
    loud = run_attention(wl)
    assert torch.equal(loud[a:b], base[a:b])


def test_sample_permutation_permutes_output_bitwise():
    w = workloads.make_workload("mixed", seed=21)
    base = run_attention(w)
    cu = np.concatenate([[0], np.cumsum(w.text_len + w.grid_hw[:, 0] * w.grid_hw[:, 1])])
    perm = [3, 0, 4, 2, 1]
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in perm])
    wp = workloads.Workload("perm", w.grid_hw[perm], w.text_len[perm], w.heads, w.head_dim, w.dtype,
                            w.q[idx], w.k[idx], w.v[idx])
    got = run_attention(wp)
    assert torch.equal(got, base[torch.from_numpy(idx).cuda()])


def test_deterministic_and_guard_band():
    w = workloads.make_workload("1024sq")
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    n = q.numel()
    guard = 4096
    buf = torch.full((n + guard,), 12345.0, dtype=torch.bfloat16, device="cuda")
    out = buf[:n].view(q.shape)
    a = binding.attn_packed(q, k, v, cu, grid, text, out=out).clone()
    b = binding.attn_packed(q, k, v, cu, grid, text)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.all(buf[n:] == 12345.0)


def test_workspace_variant_matches():
    w = workloads.make_workload("mixed", seed=22)
    q, k, v, grid, text = device_inputs(w)
    cu, _, _ = binding.build_metadata(grid, text, w.tokens)
    ref = binding.attn_packed(q, k, v, cu, grid, text)
    nbytes = binding.workspace_bytes(w.tokens, w.heads, w.head_dim, torch.bfloat16, w.n_seg)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    got = binding.attn_packed_ws(q, k, v, cu, grid, text, ws)
    assert binding.get_workspace_error(ws) == binding.MF_OK
    assert torch.equal(got, ref)
    small = torch.empty(nbytes - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.MFError) as e:
        binding.attn_packed_ws(q, k, v, cu, grid, text, small)
    assert e.value.code == binding.MF_ERR_INVALID_ARG


def test_concurrent_streams_with_separate_workspaces():
    """Two batches on two side streams at once, each with its own workspace
    (the documented rule for concurrent calls on one device): every result
    equals an eager call on the default stream bit for bit, and each
    workspace reports its own status."""
    wa = workloads.make_workload("mixed", seed=22)
    wb = workloads.make_custom([[64, 64]], [256], heads=4, head_dim=128, dtype="bf16", seed=41, name="b")
    print(f"two streams: T={wa.tokens} and T={wb.tokens}", flush=True)
    ins = []
    for w in (wa, wb):
        q, k, v, grid, text = device_inputs(w)
        cu, _, _ = binding.build_metadata(grid, text, w.tokens)
        ref = binding.attn_packed(q, k, v, cu, grid, text)
        ws = torch.empty(binding.workspace_bytes(w.tokens, w.heads, w.head_dim, torch.bfloat16, w.n_seg),
                         dtype=torch.uint8, device="cuda")
        ins.append((q, k, v, cu, grid, text, ref, ws, torch.empty_like(q)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(5):
        for s, (q, k, v, cu, grid, text, _, ws, out) in zip(streams, ins):
            with torch.cuda.stream(s):
                binding.attn_packed_ws(q, k, v, cu, grid, text, ws, out=out, stream=s)
    torch.cuda.synchronize()
    for s, (*_, ref, ws, out) in zip(streams, ins):
        assert binding.get_workspace_error(ws, s) == binding.MF_OK
        assert torch.equal(out, ref)


def test_metadata_mismatch_writes_nothing():
    w = workloads.make_custom([[4, 4], [3, 5]], [2, 1], heads=2, head_dim=128, dtype="bf16", seed=2)
    q, k, v, grid, text = device_inputs(w)
    bad_cu = torch.tensor([0, 17, w.tokens], dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    binding.attn_packed(q, k, v, bad_cu, grid, text, out=out)
    assert binding.get_device_error() == binding.MF_ERR_METADATA
    assert torch.all(out == 7.0)
    # a consistent call afterwards succeeds and clears the flag
    run_attention(w)
