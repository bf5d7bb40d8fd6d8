"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
examples (tests/golden), closed forms, invariants, special cases that reduce
to a textbook result, brute force on tiny inputs, and finite differences.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, packing, rectified_flow, rope
from text_image_diffusion_varlen_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- packing

def test_joint_pack_hand_example():
    """Labelled rows through the joint layout, worked by hand (tests/golden)."""
    g = _golden("joint_pack_small.json")
    ts = np.array(g["text_stream"]).reshape(-1, 1)
    im = np.array(g["image_stream"]).reshape(-1, 1)
    joint = packing.pack_joint(ts, im, g["grid_hw"], g["text_len"])
    assert joint[:, 0].tolist() == g["joint"]
    t2, i2 = packing.unpack_joint(np.array(g["joint"]).reshape(-1, 1), g["grid_hw"], g["text_len"])
    assert t2[:, 0].tolist() == g["text_stream"] and i2[:, 0].tolist() == g["image_stream"]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_joint_pack_agrees_with_token_positions(seed):
    """Every joint row comes from the stream its position says: rows at a
    sample's prompt positions (u < T_i) from the text stream in order, and the
    image row p of sample i (image stream order) at grid position (p // w, p % w)
    of that sample. Rows are labelled with their stream index, so a swapped
    text/image order, an off-by-one offset or a transposed grid fails."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    grid = rng.integers(1, 7, size=(n, 2))
    text = rng.integers(0, 5, size=n)
    n_text, n_img = int(text.sum()), int((grid[:, 0] * grid[:, 1]).sum())
    ts = np.arange(n_text).reshape(-1, 1) + 10_000
    im = np.arange(n_img).reshape(-1, 1) + 20_000
    joint = packing.pack_joint(ts, im, grid, text)[:, 0]
    pos, seg = packing.token_positions(grid, text)
    cu = packing.cu_seqlens(grid, text)
    t_seen = i_seen = 0
    for i in range(n):
        h, w = int(grid[i, 0]), int(grid[i, 1])
        for u in range(int(cu[i + 1] - cu[i])):
            r = int(cu[i]) + u
            assert seg[r] == i
            if u < text[i]:
                assert joint[r] == 10_000 + t_seen
                t_seen += 1
            else:
                p = joint[r] - 20_000
                assert p == i_seen
                local = p - int((grid[:i, 0] * grid[:i, 1]).sum())
                assert (pos[r, 0], pos[r, 1]) == (local // w, local % w)
                i_seen += 1
    assert (t_seen, i_seen) == (n_text, n_img)


@pytest.mark.parametrize("seed", [3, 4])
def test_joint_pack_round_trip_and_permutation(seed):
    """unpack(pack(x)) = x for 2D and editing (frames) samples; pack is a
    permutation of the concatenated streams (every row once); an empty prompt
    stream and an all-prompt-free batch work."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 7))
    grid = rng.integers(1, 6, size=(n, 2))
    text = rng.integers(0, 4, size=n)
    frames = rng.integers(1, 4, size=n)
    for fr in (None, frames):
        n_img = int(((1 if fr is None else fr) * grid[:, 0] * grid[:, 1]).sum())
        ts = rng.standard_normal((int(text.sum()), 2, 3))
        im = rng.standard_normal((n_img, 2, 3))
        joint = packing.pack_joint(ts, im, grid, text, fr)
        assert joint.shape[0] == packing.cu_seqlens(grid, text, fr)[-1]
        t2, i2 = packing.unpack_joint(joint, grid, text, fr)
        assert np.array_equal(t2, ts) and np.array_equal(i2, im)
        rows = np.concatenate([ts, im]).reshape(-1, 6)
        assert sorted(map(tuple, joint.reshape(-1, 6))) == sorted(map(tuple, rows))
    zero = np.zeros(n, dtype=np.int64)
    im = rng.standard_normal((int((grid[:, 0] * grid[:, 1]).sum()), 4))
    assert np.array_equal(packing.pack_joint(np.zeros((0, 4)), im, grid, zero), im)


def test_packing_hand_example():
    g = _golden("packing_small.json")
    cu = packing.cu_seqlens(g["grid_hw"], g["text_len"])
    pos, seg = packing.token_positions(g["grid_hw"], g["text_len"])
    assert cu.tolist() == g["cu_seqlens"]
    assert pos.tolist() == g["pos"]
    assert seg.tolist() == g["seg_id"]


def _positions_by_enumeration(grid_hw, text_len):
    """Independent construction: emit the prompt, then walk the grid with nested loops."""
    pos, seg = [], []
    for i, ((h, w), t) in enumerate(zip(grid_hw, text_len)):
        for _ in range(t):
            pos.append((0, 0))
            seg.append(i)
        for r in range(h):
            for c in range(w):
                pos.append((r, c))
                seg.append(i)
    return pos, seg


@pytest.mark.parametrize("seed", range(6))
def test_packing_matches_enumeration(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 6))
    grid = [(int(rng.integers(1, 9)), int(rng.integers(1, 9))) for _ in range(n)]
    text = [int(rng.integers(0, 7)) for _ in range(n)]
    pos, seg = packing.token_positions(grid, text)
    pos_e, seg_e = _positions_by_enumeration(grid, text)
    assert [tuple(p) for p in pos.tolist()] == pos_e
    assert seg.tolist() == seg_e
    cu = packing.cu_seqlens(grid, text)
    # offsets are where the sample id changes
    starts = [0] + [j for j in range(1, len(seg_e)) if seg_e[j] != seg_e[j - 1]] + [len(seg_e)]
    assert cu.tolist() == starts


@pytest.mark.parametrize("config", ["tiny", "1024sq", "mixed", "2048sq", "train65k"])
def test_packing_invariants_on_configs(config):
    grid, text = workloads.make_segments(config)
    cu = packing.cu_seqlens(grid, text)
    pos, seg = packing.token_positions(grid, text)
    assert cu[0] == 0 and cu[-1] == pos.shape[0]
    assert np.all(np.diff(cu) == text + grid[:, 0] * grid[:, 1])
    for i in range(len(text)):
        a, b = cu[i], cu[i + 1]
        assert np.all(seg[a:b] == i)
        p = pos[a + text[i] : b]
        h, w = grid[i]
        assert p[:, 0].max() < h and p[:, 1].max() < w and p.min() >= 0
        # every grid cell exactly once
        cells = p[:, 0].astype(np.int64) * w + p[:, 1]
        assert np.array_equal(np.sort(cells), np.arange(h * w))
        assert np.all(pos[a : a + text[i]] == 0)
    if config == "train65k":
        assert cu[-1] <= 65536


def test_packing_rejects_bad_segments():
    with pytest.raises(ValueError):
        packing.cu_seqlens([[0, 4]], [3])
    with pytest.raises(ValueError):
        packing.cu_seqlens([[2, 4]], [-1])
    with pytest.raises(ValueError):
        packing.cu_seqlens([[2, 4], [1, 1]], [3])


def test_workload_recipes():
    g, t = workloads.make_segments("mixed")
    assert g.tolist() == [[32, 128], [128, 32], [48, 84], [64, 64], [32, 32]]
    assert np.all((t >= 77) & (t <= 256))
    g, t = workloads.make_segments("train65k")
    assert np.all(g % 2 == 0) and g.min() >= 32 and g.max() <= 128
    w = workloads.make_workload("tiny")
    assert w.q.shape == (288, 2, 64) and w.dtype == "f32"
    # bf16 rounding of the generator is round-to-nearest-even
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.0 - 2**-7 * 1.5], dtype=np.float32)
    r = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x))
    assert r.tolist() == [1.0, 1.0, 1.0 + 2**-6, -2.0 - 2**-6]


# ---------------------------------------------------------------- rope

def test_rope_hand_examples():
    for case in _golden("rope_small.json")["cases"]:
        x = np.array(case["x"], dtype=np.float64).reshape(1, 1, -1)
        got = rope.rope2d(x, np.array([case["pos"]]))[0, 0]
        exp = []
        for j, phi in enumerate(case["pair_angles"]):
            x0, x1 = case["x"][2 * j], case["x"][2 * j + 1]
            exp += [x0 * math.cos(phi) - x1 * math.sin(phi), x0 * math.sin(phi) + x1 * math.cos(phi)]
        np.testing.assert_allclose(got, exp, rtol=0, atol=1e-15)


def test_rope_frequency_ladder():
    for d in (8, 64, 128):
        f = rope.axis_frequencies(d // 2)
        assert f.shape == (d // 4,)
        assert f[0] == 1.0
        ratio = f[1:] / f[:-1]
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-13)
        # one more rung of the ladder reaches exactly 1/theta
        np.testing.assert_allclose(f[-1] * ratio[0], 1.0 / 10000.0, rtol=1e-12)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_rope_is_complex_rotation(d):
    """Each channel pair, read as a complex number x0 + i x1, is multiplied by exp(i phi)."""
    x = _rand((5, 3, d), 1)
    pos = np.array([[0, 0], [1, 7], [63, 2], [127, 127], [9, 0]])
    got = rope.rope2d(x, pos)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    half = d // 4
    for t in range(5):
        for p in range(d // 2):
            axis, j = (0, p) if p < half else (1, p - half)
            phi = pos[t, axis] * 10000.0 ** (-2.0 * j / (d // 2))
            w = z[t, :, p] * np.exp(1j * phi)
            np.testing.assert_allclose(got[t, :, 2 * p], w.real, atol=1e-12)
            np.testing.assert_allclose(got[t, :, 2 * p + 1], w.imag, atol=1e-12)


def test_rope_norm_identity_inverse_composition():
    x = _rand((40, 2, 64), 2)
    rng = np.random.default_rng(3)
    p1 = rng.integers(0, 128, size=(40, 2))
    p2 = rng.integers(0, 128, size=(40, 2))
    r = rope.rope2d(x, p1)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(rope.rope2d(x, np.zeros_like(p1)), x)
    np.testing.assert_allclose(rope.rope2d_inverse(r, p1), x, atol=1e-12)
    np.testing.assert_allclose(rope.rope2d(r, p2), rope.rope2d(x, p1 + p2), atol=1e-11)


def test_rope_relative_position_invariance():
    """R(p) q . R(p') k depends only on p - p' (a shared integer shift changes nothing)."""
    q = _rand((30, 2, 128), 4)
    k = _rand((30, 2, 128), 5)
    rng = np.random.default_rng(6)
    pq = rng.integers(0, 100, size=(30, 2))
    pk = rng.integers(0, 100, size=(30, 2))
    base = np.einsum("thd,shd->tsh", rope.rope2d(q, pq), rope.rope2d(k, pk))
    for shift in ([5, 0], [0, 11], [17, 23]):
        s = np.array(shift)
        moved = np.einsum("thd,shd->tsh", rope.rope2d(q, pq + s), rope.rope2d(k, pk + s))
        np.testing.assert_allclose(moved, base, atol=1e-10)
    # and it is not invariant to a shift of only one side (the rotation does something)
    moved = np.einsum("thd,shd->tsh", rope.rope2d(q, pq + 3), rope.rope2d(k, pk))
    assert np.abs(moved - base).max() > 1e-2


def test_rope_reduces_to_1d_on_a_single_row():
    """On a 1 x w grid the row half is untouched and the column half is ordinary 1D RoPE
    over d/2 channels (pair j at angle col * theta^(-2j/(d/2)))."""
    d = 64
    x = _rand((12, 2, d), 7)
    pos = np.stack([np.zeros(12, int), np.arange(12)], axis=1)
    got = rope.rope2d(x, pos)
    np.testing.assert_array_equal(got[..., : d // 2], x[..., : d // 2])
    xb = x[..., d // 2 :]
    z = xb[..., 0::2] + 1j * xb[..., 1::2]
    m = d // 2
    inv = 10000.0 ** (-np.arange(0, m, 2) / m)
    w = z * np.exp(1j * np.arange(12)[:, None, None] * inv[None, None, :])
    np.testing.assert_allclose(got[..., d // 2 :: 2], w.real, atol=1e-12)
    np.testing.assert_allclose(got[..., d // 2 + 1 :: 2], w.imag, atol=1e-12)


def test_rope3d_reduces_to_2d_at_frame_zero():
    x = _rand((10, 2, 16), 8)
    rng = np.random.default_rng(9)
    p = rng.integers(0, 50, size=(10, 2))
    p3 = np.concatenate([p, np.zeros((10, 1), int)], axis=1)
    # row/col blocks of 8 channels and an empty frame block: identical to rope2d
    np.testing.assert_allclose(rope.rope3d(x, p3, (8, 8, 0)), rope.rope2d(x, p), atol=1e-14)
    # the frame block only turns when the frame index changes
    y = rope.rope3d(x, p3, (4, 4, 8))
    np.testing.assert_array_equal(y[..., 8:], x[..., 8:])
    p3[:, 2] = 1
    assert np.abs(rope.rope3d(x, p3, (4, 4, 8))[..., 8:] - x[..., 8:]).max() > 1e-3


# ---------------------------------------------------------------- attention

def _brute_attention(q, k, v, scale):
    """Triple loop in pure Python floats: no BLAS, no vectorization."""
    L, H, d = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * len(v[0][0]) for _ in range(H)] for _ in range(L)]
    for h in range(H):
        for i in range(L):
            s = [sum(q[i][h][c] * k[j][h][c] for c in range(d)) * scale for j in range(len(k))]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for c in range(len(v[0][0])):
                out[i][h][c] = sum(e[j] * v[j][h][c] for j in range(len(k))) / z
    return out


def test_attention_hand_example():
    g = _golden("attention_small.json")
    q = np.array(g["q"])[:, None, :]
    k = np.array(g["k"])[:, None, :]
    v = np.array(g["v"])[:, None, :]
    got = attention.sample_attention(q, k, v)[:, 0, :]
    np.testing.assert_allclose(got, g["out"], atol=1e-12)


@pytest.mark.parametrize("L,H,d", [(1, 1, 4), (7, 2, 8), (23, 2, 16)])
def test_attention_matches_brute_force(L, H, d):
    rng = np.random.default_rng(L * 31 + d)
    q, k, v = (rng.standard_normal((L, H, d)) for _ in range(3))
    got = attention.sample_attention(q, k, v, row_block=5)
    exp = _brute_attention(q.tolist(), k.tolist(), v.tolist(), 1.0 / math.sqrt(d))
    np.testing.assert_allclose(got, np.array(exp), atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(11)
    q, v = rng.standard_normal((9, 2, 8)), rng.standard_normal((9, 2, 8))
    # zero keys: uniform weights -> mean of v
    got = attention.sample_attention(q, np.zeros_like(q), v)
    np.testing.assert_allclose(got, np.broadcast_to(v.mean(axis=0), v.shape), atol=1e-13)
    # constant values: output is that constant
    c = np.broadcast_to(rng.standard_normal((1, 2, 8)), v.shape)
    got = attention.sample_attention(q, rng.standard_normal(q.shape), c)
    np.testing.assert_allclose(got, c, atol=1e-13)
    # a single token attends only to itself
    got = attention.sample_attention(q[:1], q[:1] * 3, v[:1])
    np.testing.assert_allclose(got, v[:1], atol=0)
    # two keys: weight of key 0 is the logistic function of the score gap
    k2 = rng.standard_normal((2, 1, 8))
    v2 = np.array([[[1.0] * 8], [[0.0] * 8]])
    q1 = rng.standard_normal((3, 1, 8))
    got = attention.sample_attention(q1, k2, v2)[:, 0, 0]
    gap = (q1[:, 0] @ (k2[0, 0] - k2[1, 0])) / math.sqrt(8)
    np.testing.assert_allclose(got, 1.0 / (1.0 + np.exp(-gap)), atol=1e-14)


def test_attention_sharp_limit_is_argmax():
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((6, 1, 8)) for _ in range(3))
    got = attention.sample_attention(q, k, v, scale=1e4)
    best = np.argmax(q[:, 0] @ k[:, 0].T, axis=1)
    np.testing.assert_allclose(got[:, 0], v[best, 0], atol=1e-9)


def test_attention_permutation_rules():
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((15, 2, 8)) for _ in range(3))
    base = attention.sample_attention(q, k, v)
    perm = rng.permutation(15)
    np.testing.assert_allclose(attention.sample_attention(q, k[perm], v[perm]), base, atol=1e-13)
    np.testing.assert_allclose(attention.sample_attention(q[perm], k, v), base[perm], atol=1e-13)


def test_packed_equals_masked_dense():
    grid, text = [[3, 4], [1, 1], [2, 5], [4, 1]], [2, 0, 5, 3]
    cu = packing.cu_seqlens(grid, text)
    _, seg = packing.token_positions(grid, text)
    rng = np.random.default_rng(14)
    T = int(cu[-1])
    q, k, v = (rng.standard_normal((T, 2, 8)) for _ in range(3))
    np.testing.assert_allclose(
        attention.packed_attention(q, k, v, cu), attention.masked_attention(q, k, v, seg), atol=1e-13)
    # a sample's output does not depend on the other samples' contents
    k2 = k.copy()
    k2[cu[1] :] = rng.standard_normal(k2[cu[1] :].shape)
    a = attention.packed_attention(q, k, v, cu)
    b = attention.packed_attention(q, k2, v, cu)
    np.testing.assert_array_equal(a[: cu[1]], b[: cu[1]])


def test_joint_attention_pipeline_small():
    """Full path = explicit rotation + masked dense attention, on the hand-worked packing."""
    g = _golden("packing_small.json")
    rng = np.random.default_rng(15)
    T = g["cu_seqlens"][-1]
    q, k, v = (rng.standard_normal((T, 2, 8)) for _ in range(3))
    got = attention.joint_attention(q, k, v, g["grid_hw"], g["text_len"])
    pos = np.array(g["pos"])
    exp = attention.masked_attention(rope.rope2d(q, pos), rope.rope2d(k, pos), v, np.array(g["seg_id"]))
    np.testing.assert_allclose(got, exp, atol=1e-13)
    rows = [0, 5, 9, 13]
    np.testing.assert_allclose(
        attention.joint_attention_rows(q, k, v, g["grid_hw"], g["text_len"], rows), got[rows], atol=1e-13)


def test_joint_attention_image_only_shift_invariance():
    """With no prompt tokens every position is an image position; a common shift of
    all of them leaves the attention output unchanged (relative RoPE)."""
    grid, text = [[3, 5]], [0]
    rng = np.random.default_rng(16)
    q, k, v = (rng.standard_normal((15, 2, 16)) for _ in range(3))
    base = attention.joint_attention(q, k, v, grid, text)
    pos, _ = packing.token_positions(grid, text)
    cu = packing.cu_seqlens(grid, text)
    moved = pos + np.array([7, 4])
    got = attention.packed_attention(rope.rope2d(q, moved), rope.rope2d(k, moved), v, cu)
    np.testing.assert_allclose(got, base, atol=1e-12)


def test_lse_matches_brute_force():
    rng = np.random.default_rng(17)
    q, k = rng.standard_normal((5, 1, 4)), rng.standard_normal((7, 1, 4))
    lse = attention.sample_attention_lse(q, k)
    for i in range(5):
        s = [float(q[i, 0] @ k[j, 0]) / 2.0 for j in range(7)]
        assert abs(lse[i, 0] - math.log(sum(math.exp(x) for x in s))) < 1e-12


def test_joint_lse_brute_force_with_complex_rotation():
    """Joint LSE against a pure-Python evaluation: positions enumerated by hand,
    each channel pair rotated as a complex number times e^{i p w_j}, scores and
    log-sum-exp summed term by term per sample."""
    grid, text = [[2, 3], [1, 2]], [2, 1]
    d, H = 8, 2
    rng = np.random.default_rng(21)
    T = sum(t + h * w for (h, w), t in zip(grid, text))
    q, k = rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d))
    lse = attention.joint_attention_lse(q, k, grid, text)
    samples, start = [], 0
    for (h, w), t in zip(grid, text):
        pos = [(0, 0)] * t + [(r, c) for r in range(h) for c in range(w)]
        samples.append((start, pos))
        start += t + h * w

    def rot(x, p):
        out = []
        for j in range(d // 2):
            half, jj = divmod(j, d // 4)
            ang = p[half] * 10000.0 ** (-2 * jj / (d // 2))
            z = complex(x[2 * j], x[2 * j + 1]) * complex(math.cos(ang), math.sin(ang))
            out += [z.real, z.imag]
        return out

    for start, pos in samples:
        n = len(pos)
        for hh in range(H):
            qr = [rot(q[start + i, hh], pos[i]) for i in range(n)]
            kr = [rot(k[start + i, hh], pos[i]) for i in range(n)]
            for i in range(n):
                s = [sum(a * b for a, b in zip(qr[i], kr[j])) / math.sqrt(d) for j in range(n)]
                assert abs(lse[hh, start + i] - math.log(sum(math.exp(x) for x in s))) < 1e-12


def _numeric_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    for idx in itertools.product(*map(range, x.shape)):
        xp = x.copy()
        xp[idx] += eps
        xm = x.copy()
        xm[idx] -= eps
        g[idx] = (f(xp) - f(xm)) / (2 * eps)
    return g


def test_attention_backward_finite_differences():
    grid, text = [[2, 2], [1, 3]], [1, 2]
    T = 10
    rng = np.random.default_rng(18)
    q, k, v, w = (rng.standard_normal((T, 2, 4)) for _ in range(4))

    def loss(qq, kk, vv):
        return float(np.sum(attention.joint_attention(qq, kk, vv, grid, text) * w))

    dq, dk, dv = attention.joint_attention_backward(q, k, v, w, grid, text)
    np.testing.assert_allclose(dq, _numeric_grad(lambda x: loss(x, k, v), q), atol=1e-7)
    np.testing.assert_allclose(dk, _numeric_grad(lambda x: loss(q, x, v), k), atol=1e-7)
    np.testing.assert_allclose(dv, _numeric_grad(lambda x: loss(q, k, x), v), atol=1e-7)


# ---------------------------------------------------------------- rectified flow

def test_rf_hand_example():
    g = _golden("rf_small.json")
    np.testing.assert_array_equal(rectified_flow.interpolate(g["z0"], g["z1"], g["t"]), g["z_t"])
    np.testing.assert_array_equal(rectified_flow.target_velocity(g["z0"], g["z1"]), g["velocity"])
    assert rectified_flow.interpolate(g["z0"], g["z1"], 0.0).tolist() == g["z0"]
    assert rectified_flow.interpolate(g["z0"], g["z1"], 1.0).tolist() == g["z1"]


@pytest.mark.parametrize("steps", [1, 4, 20, 30])
def test_rf_euler_follows_the_straight_path(steps):
    rng = np.random.default_rng(19)
    z0, z1 = rng.standard_normal((2, 3, 8)), rng.standard_normal((2, 3, 8))
    grid = rectified_flow.uniform_grid(steps)
    fields = [lambda z, t: z1 - z0, lambda z, t: (z1 - z) / (1.0 - t)]
    for field in fields:
        for solver in (rectified_flow.euler, rectified_flow.midpoint):
            states = solver(z0, field, grid)
            for t, z in zip(grid, states):
                np.testing.assert_allclose(z, t * z1 + (1 - t) * z0, atol=1e-12)
            np.testing.assert_allclose(states[-1], z1, atol=1e-12)


def test_rf_euler_is_inexact_on_a_curved_field():
    """A field that is not constant along the path (v = -z, exact flow z0 e^{-t}): one
    Euler step lands at z0 (1 - dt) per step, not on the exponential -- the solver is
    genuinely stepping, not returning a closed form."""
    z0 = np.array([1.0])
    st = rectified_flow.euler(z0, lambda z, t: -z, rectified_flow.uniform_grid(4))
    np.testing.assert_allclose(st[-1], [0.75**4], atol=1e-15)
    st = rectified_flow.midpoint(z0, lambda z, t: -z, rectified_flow.uniform_grid(4))
    np.testing.assert_allclose(st[-1], [(1 - 0.25 + 0.25**2 / 2) ** 4], atol=1e-15)


def test_rf_loss_and_cfg():
    rng = np.random.default_rng(20)
    z0, z1 = rng.standard_normal((4, 6)), rng.standard_normal((4, 6))
    assert rectified_flow.loss(z1 - z0, z0, z1) == 0.0
    np.testing.assert_allclose(rectified_flow.loss(np.zeros_like(z0), z0, z1),
                               np.mean(np.sum((z1 - z0) ** 2, axis=1)), rtol=1e-14)
    vu, vc = rng.standard_normal((2, 5))
    np.testing.assert_allclose(rectified_flow.cfg_combine(vu, vc, 0.0), vu)
    np.testing.assert_allclose(rectified_flow.cfg_combine(vu, vc, 1.0), vc, atol=1e-15)
    np.testing.assert_allclose(rectified_flow.cfg_combine(vu, vc, 5.0), 5 * vc - 4 * vu, atol=1e-13)


# ---------------------------------------------------------------- packed CFG step

from cfg_common import guided_field  # noqa: E402


@pytest.mark.parametrize("layout", ["interleaved", "blocks", "shuffled"])
@pytest.mark.parametrize("guidance", [5.0, 1.0, -2.0])
def test_packed_cfg_euler_lands_on_data(layout, guidance):
    """Four guided Euler steps along the constructed field follow the straight
    path t z1 + (1 - t) z0 and land on z1 (closed form of the straight path)."""
    batch = workloads.make_cfg_batch([(3, 5), (1, 1), (4, 2), (2, 7)], [4, 0, 9, 2], [0, 3, 1, 0], layout,
                                     channels=8, dtype="f32", seed=11, guided=[1, 1, 0, 1])
    rng = np.random.default_rng(12)
    z0 = batch.z.astype(np.float64)
    z1 = rng.standard_normal(z0.shape)
    z = z0
    grid = rectified_flow.uniform_grid(4)
    for k in range(4):
        t, dt = grid[k], grid[k + 1] - grid[k]
        v = guided_field(batch, z, z1, t, guidance, rng.standard_normal(batch.v.shape))
        z = rectified_flow.packed_cfg_euler_step(z, v, batch.grid_hw, batch.text_len, batch.cond_seg,
                                                 batch.uncond_seg, guidance, dt)
        np.testing.assert_allclose(z, grid[k + 1] * z1 + (1 - grid[k + 1]) * z0, atol=1e-12)
    np.testing.assert_allclose(z, z1, atol=1e-12)


def test_packed_cfg_euler_special_cases():
    batch = workloads.make_cfg_batch([(3, 4), (2, 2)], [5, 1], [2, 0], "shuffled", channels=8, dtype="f32",
                                     seed=13)
    args = (batch.grid_hw, batch.text_len, batch.cond_seg, batch.uncond_seg)
    step = rectified_flow.packed_cfg_euler_step
    z, v = batch.z, batch.v
    # dt = 0 leaves z alone; text rows never matter
    np.testing.assert_array_equal(step(z, v, *args, 5.0, 0.0), z)
    v2 = v.copy()
    run = 0
    for (h, w), t in zip(batch.grid_hw.tolist(), batch.text_len.tolist()):
        v2[run:run + t] = 1e6
        run += t + h * w
    np.testing.assert_array_equal(step(z, v2, *args, 5.0, 0.5), step(z, v, *args, 5.0, 0.5))
    # guidance 0 / no unconditional sample: the unguided step of the matching branch
    nog = np.full_like(batch.uncond_seg, -1)
    a = step(z, v, batch.grid_hw, batch.text_len, batch.uncond_seg, nog, 7.0, 0.5)
    np.testing.assert_allclose(step(z, v, *args, 0.0, 0.5), a, atol=1e-14)
    c = step(z, v, batch.grid_hw, batch.text_len, batch.cond_seg, nog, 7.0, 0.5)
    np.testing.assert_allclose(step(z, v, *args, 1.0, 0.5), c, atol=1e-14)
    # the step is affine in dt
    d1, d2 = step(z, v, *args, 3.0, 0.25) - z, step(z, v, *args, 3.0, 0.75) - z
    np.testing.assert_allclose(3 * d1, d2, atol=1e-13)


# ---------------------------------------------------------------- frame-aware (editing) variant


def test_positions_3d_enumeration():
    grid, text, frames = [[2, 3], [1, 1], [3, 2]], [2, 0, 1], [2, 3, 1]
    pos3, seg = packing.token_positions_3d(grid, text, frames)
    exp, eseg = [], []
    for i, ((h, w), t, f) in enumerate(zip(grid, text, frames)):
        for _ in range(t):
            exp.append((0, 0, 0))
            eseg.append(i)
        for fr in range(f):
            for r in range(h):
                for c in range(w):
                    exp.append((r, c, fr))
                    eseg.append(i)
    assert pos3.tolist() == [list(x) for x in exp]
    assert seg.tolist() == eseg
    assert packing.cu_seqlens(grid, text, frames).tolist() == [0, 14, 17, 24]
    # one image per sample: the 2D positions at frame 0
    p2, s2 = packing.token_positions(grid, text)
    p1, s1 = packing.token_positions_3d(grid, text, [1, 1, 1])
    assert np.array_equal(p1[:, :2], p2) and not p1[:, 2].any() and np.array_equal(s1, s2)


@pytest.mark.parametrize("split", [(4, 6, 6), (8, 4, 4), (6, 6, 4)])
def test_rope3d_is_complex_rotation(split):
    d = 16
    rng = np.random.default_rng(40)
    x = rng.standard_normal((5, 2, d))
    p3 = rng.integers(0, 40, size=(5, 3))
    y = rope.rope3d(x, p3, split)
    bounds = np.cumsum([0] + list(split))
    for t in range(5):
        for a in range(3):
            m = split[a]
            for j in range(m // 2):
                ch = bounds[a] + 2 * j
                ang = p3[t, a] * 10000.0 ** (-2.0 * j / m)
                z = (x[t, :, ch] + 1j * x[t, :, ch + 1]) * np.exp(1j * ang)
                np.testing.assert_allclose(y[t, :, ch], z.real, atol=1e-12)
                np.testing.assert_allclose(y[t, :, ch + 1], z.imag, atol=1e-12)
    np.testing.assert_allclose(rope.rope3d_inverse(y, p3, split), x, atol=1e-12)


def test_rope3d_relative_in_every_axis():
    rng = np.random.default_rng(41)
    q, k = rng.standard_normal((2, 1, 1, 24))
    for delta in ([0, 0, 3], [2, 5, 0], [7, 1, 9]):
        p, pp = np.array([[3, 4, 1]]), np.array([[1, 9, 2]])
        a = np.sum(rope.rope3d(q, p, (8, 8, 8)) * rope.rope3d(k, pp, (8, 8, 8)))
        b = np.sum(rope.rope3d(q, p + delta, (8, 8, 8)) * rope.rope3d(k, pp + delta, (8, 8, 8)))
        assert abs(a - b) < 1e-12


def test_joint_attention_3d_reduces_to_2d():
    grid, text = [[3, 4], [2, 2]], [5, 0]
    rng = np.random.default_rng(42)
    T = 5 + 12 + 4
    q, k, v = (rng.standard_normal((T, 2, 8)) for _ in range(3))
    a = attention.joint_attention(q, k, v, grid, text)
    b = attention.joint_attention_3d(q, k, v, grid, text, [1, 1], (4, 4, 0))
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_joint_attention_3d_brute_force():
    """Output and LSE of a two-image editing sample against pure-Python loops
    (complex rotation per channel pair, explicit softmax)."""
    grid, text, frames, split = [[2, 2], [1, 3]], [2, 1], [2, 3], (2, 2, 4)
    d, H = 8, 1
    rng = np.random.default_rng(43)
    T = 2 + 8 + 1 + 9
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    out = attention.joint_attention_3d(q, k, v, grid, text, frames, split)
    lse = attention.joint_attention_3d_lse(q, k, grid, text, frames, split)

    def rot(x, p):
        res, base = [], 0
        for a, m in enumerate(split):
            for j in range(m // 2):
                z = complex(x[base + 2 * j], x[base + 2 * j + 1]) * complex(
                    math.cos(p[a] * 10000.0 ** (-2 * j / m)), math.sin(p[a] * 10000.0 ** (-2 * j / m)))
                res += [z.real, z.imag]
            base += m
        return res

    start = 0
    for (h, w), t, f in zip(grid, text, frames):
        pos = [(0, 0, 0)] * t + [(r, c, fr) for fr in range(f) for r in range(h) for c in range(w)]
        n = len(pos)
        qr = [rot(q[start + i, 0], pos[i]) for i in range(n)]
        kr = [rot(k[start + i, 0], pos[i]) for i in range(n)]
        for i in range(n):
            s = [sum(a * b for a, b in zip(qr[i], kr[j])) / math.sqrt(d) for j in range(n)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            assert abs(lse[0, start + i] - (m + math.log(z))) < 1e-12
            for c in range(d):
                ref = sum(e[j] * v[start + j, 0, c] for j in range(n)) / z
                assert abs(out[start + i, 0, c] - ref) < 1e-12
        start += n


def test_attention_3d_backward_finite_differences():
    grid, text, frames, split = [[1, 2], [2, 1]], [1, 0], [2, 2], (2, 2, 4)
    T = 5 + 4
    rng = np.random.default_rng(44)
    q, k, v, w = (rng.standard_normal((T, 1, 8)) for _ in range(4))

    def loss(qq, kk, vv):
        return float(np.sum(attention.joint_attention_3d(qq, kk, vv, grid, text, frames, split) * w))

    dq, dk, dv = attention.joint_attention_3d_backward(q, k, v, w, grid, text, frames, split)
    np.testing.assert_allclose(dq, _numeric_grad(lambda x: loss(x, k, v), q), atol=1e-7)
    np.testing.assert_allclose(dk, _numeric_grad(lambda x: loss(q, x, v), k), atol=1e-7)
    np.testing.assert_allclose(dv, _numeric_grad(lambda x: loss(q, k, x), v), atol=1e-7)


# ---------------------------------------------------------------- RMSNorm + packed QKV

from oracle import projection  # noqa: E402


def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(70)
    x = rng.standard_normal((6, 32))
    h = projection.rmsnorm(x, np.ones(32), eps=0.0)
    np.testing.assert_allclose(np.mean(h * h, axis=-1), 1.0, atol=1e-14)   # unit RMS
    np.testing.assert_allclose(projection.rmsnorm(7.5 * x, np.ones(32), eps=0.0), h, atol=1e-13)  # scale-free
    ms = np.mean(x * x, axis=-1)
    he = projection.rmsnorm(x, np.ones(32), eps=0.25)
    np.testing.assert_allclose(np.mean(he * he, axis=-1), ms / (ms + 0.25), atol=1e-14)
    g = rng.standard_normal(32)
    np.testing.assert_allclose(projection.rmsnorm(x, g, eps=0.0), h * g, atol=1e-14)
    # a constant row c: sqrt(c^2) = |c|, so the row becomes sign(c) * gamma
    np.testing.assert_allclose(projection.rmsnorm(np.full((1, 4), -3.0), [1, 2, 3, 4], eps=0.0), [[-1, -2, -3, -4]])


def test_rmsnorm_qkv_brute_force_and_routing():
    grid, text, heads, d = [[2, 2], [1, 3]], [3, 1], 2, 4
    C, hd = 8, heads * d
    T = 3 + 4 + 1 + 3
    rng = np.random.default_rng(71)
    x = rng.standard_normal((T, C))
    wt, wi = rng.standard_normal((3 * hd, C)), rng.standard_normal((3 * hd, C))
    gt, gi = rng.standard_normal(C), rng.standard_normal(C)
    q, k, v = projection.rmsnorm_qkv(x, wt, wi, gt, gi, grid, text, heads, d)
    is_text = [True] * 3 + [False] * 4 + [True] + [False] * 3
    for t in range(T):
        w, g = (wt, gt) if is_text[t] else (wi, gi)
        r = math.sqrt(sum(float(a) ** 2 for a in x[t]) / C + 1e-6)
        hrow = [float(x[t, c]) / r * float(g[c]) for c in range(C)]
        for which, out in enumerate((q, k, v)):
            for h in range(heads):
                for j in range(d):
                    n = which * hd + h * d + j
                    ref = sum(hrow[c] * float(w[n, c]) for c in range(C))
                    assert abs(out[t, h, j] - ref) < 1e-12
    # zero visual weights: visual rows vanish, text rows do not
    q0, _, _ = projection.rmsnorm_qkv(x, wt, np.zeros_like(wi), gt, gi, grid, text, heads, d)
    assert not q0[~np.array(is_text)].any() and q0[np.array(is_text)].any()


def test_text_mask_editing_samples():
    m = projection.text_mask([[1, 2], [2, 1]], [2, 0], [3, 2])
    assert m.tolist() == [True, True] + [False] * 6 + [False] * 4
