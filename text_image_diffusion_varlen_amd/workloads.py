"""Seeded synthetic workloads for packed joint text+image attention.

This module only draws random numbers. It holds none of the attention, RoPE or
packing arithmetic, so both the GPU path and the CPU oracle can consume its
output without sharing any of the method's code.

A workload is a list of segments. Segment i is one prompt of ``text_len[i]``
tokens followed by one image whose latent grid is ``grid_hw[i] = (h, w)`` at
16 px per latent token (the VAE downsamples 16x with 128 channels: Mage-Flow
tech report, Mage-VAE section; the 2x2 latent patches of the mageflow.net
architecture page, section 2, give the same 16 px). Q, K and V are
``[tokens, heads, head_dim]`` row-major in the packed (concatenated) order.

bf16 inputs are drawn as float32 N(0, 1) and rounded to bf16 with
round-to-nearest-even. Both sides read exactly those bf16 values; the float32
view returned here holds them exactly.

Random draws come in a fixed order per seed: segment metadata first, then q,
k, v, each as ``standard_normal((T, H, d), float32)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "CONFIGS",
    "make_workload",
    "make_segments",
    "make_custom",
    "EDIT_CONFIGS",
    "make_qkv_inputs",
    "make_edit",
    "CfgBatch",
    "CFG_CONFIGS",
    "make_cfg_batch",
    "make_cfg_config",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]

# Packing budget of the training-style block (tokens per packed block).
TRAIN_TOKEN_BUDGET = 65536


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs are finite here.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    rounded = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One packed batch: segment metadata plus Q/K/V of the joint sequence."""

    name: str
    grid_hw: np.ndarray  # int32 [n, 2], (h, w) latent grid of each image
    text_len: np.ndarray  # int32 [n], prompt tokens of each segment
    heads: int
    head_dim: int
    dtype: str  # "bf16" or "f32"
    q: np.ndarray = field(repr=False)  # float32 [T, H, d], exactly representable in dtype
    k: np.ndarray = field(repr=False)
    v: np.ndarray = field(repr=False)
    seed: int = 0
    frames: np.ndarray | None = None  # int32 [n]: images per editing sample (None: one image each)
    rope_split: tuple | None = None   # (row, col, frame) channels of the frame-aware RoPE

    @property
    def n_seg(self) -> int:
        return int(self.grid_hw.shape[0])

    @property
    def tokens(self) -> int:
        return int(self.q.shape[0])

    def bits(self, name: str) -> np.ndarray:
        """bf16 bit patterns (uint16) of q, k or v; only for bf16 workloads."""
        if self.dtype != "bf16":
            raise ValueError("bit patterns exist only for bf16 workloads")
        return f32_to_bf16_bits(getattr(self, name))


def _draw_train_segments(rng: np.random.Generator, budget: int):
    """Training-style block: images of independent H, W in multiples of 32 px in
    [512, 2048], prompt length uniform in [77, 256], appended until the next
    sample would exceed the token budget (that sample is dropped)."""
    grids, texts, used = [], [], 0
    while True:
        h = int(rng.integers(16, 65)) * 2  # 32 px multiples -> grid side = px / 16
        w = int(rng.integers(16, 65)) * 2
        t = int(rng.integers(77, 257))
        if used + t + h * w > budget:
            break
        grids.append((h, w))
        texts.append(t)
        used += t + h * w
    return grids, texts


# name -> (segment recipe, heads, head_dim, dtype, value scale, default seed)
CONFIGS = {
    # One 256x256 image (16x16 grid) and a 32-token prompt, fp32, 2 heads x 64.
    "tiny": dict(grids=[(16, 16)], texts=[32], heads=2, head_dim=64, dtype="f32", scale=1.0 / 8.0, seed=0),
    # One 1024x1024 image (64x64 grid) and a 256-token prompt.
    "1024sq": dict(grids=[(64, 64)], texts=[256], heads=24, head_dim=128, dtype="bf16", scale=1.0, seed=1),
    # Five mixed-aspect images, prompt lengths drawn uniformly in [77, 256].
    "mixed": dict(
        grids=[(32, 128), (128, 32), (48, 84), (64, 64), (32, 32)],
        texts="draw",
        heads=24,
        head_dim=128,
        dtype="bf16",
        scale=1.0,
        seed=2,
    ),
    # One 2048x2048 image (128x128 grid) and a 256-token prompt.
    "2048sq": dict(grids=[(128, 128)], texts=[256], heads=24, head_dim=128, dtype="bf16", scale=1.0, seed=3),
    # Training-style packed block under a 65536-token budget.
    "train65k": dict(grids="train", texts="train", heads=24, head_dim=128, dtype="bf16", scale=1.0, seed=4),
}


def make_segments(config: str, seed: int | None = None):
    """Draw only the segment metadata of a config: (grid_hw int32 [n,2], text_len int32 [n])."""
    c = CONFIGS[config]
    seed = c["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    grids, texts = _segments_from_rng(c, rng)
    return np.asarray(grids, dtype=np.int32).reshape(-1, 2), np.asarray(texts, dtype=np.int32)


def _segments_from_rng(c, rng):
    if c["grids"] == "train":
        return _draw_train_segments(rng, TRAIN_TOKEN_BUDGET)
    grids = list(c["grids"])
    if c["texts"] == "draw":
        texts = [int(rng.integers(77, 257)) for _ in grids]
    else:
        texts = list(c["texts"])
    return grids, texts


def _draw_qkv(rng, n_tokens, heads, head_dim, dtype, scale):
    out = []
    for _ in range(3):
        x = rng.standard_normal((n_tokens, heads, head_dim), dtype=np.float32)
        if scale != 1.0:
            x = (x * np.float32(scale)).astype(np.float32)
        if dtype == "bf16":
            x = bf16_bits_to_f32(f32_to_bf16_bits(x))
        out.append(np.ascontiguousarray(x))
    return out


def make_workload(config: str, seed: int | None = None) -> Workload:
    """Build the seeded workload of a named config."""
    c = CONFIGS[config]
    seed = c["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    grids, texts = _segments_from_rng(c, rng)
    grid_hw = np.asarray(grids, dtype=np.int32).reshape(-1, 2)
    text_len = np.asarray(texts, dtype=np.int32)
    # Buffer size only: every segment contributes its prompt and its image grid.
    n_tokens = int(text_len.astype(np.int64).sum() + (grid_hw[:, 0].astype(np.int64) * grid_hw[:, 1]).sum())
    q, k, v = _draw_qkv(rng, n_tokens, c["heads"], c["head_dim"], c["dtype"], c["scale"])
    return Workload(config, grid_hw, text_len, c["heads"], c["head_dim"], c["dtype"], q, k, v, seed)


def make_custom(grid_hw, text_len, heads, head_dim, dtype="bf16", seed=0, scale=1.0, name="custom") -> Workload:
    """Workload from explicit segments (used for edge cases: empty prompts, 1-wide grids, ragged tails)."""
    grid_hw = np.asarray(grid_hw, dtype=np.int32).reshape(-1, 2)
    text_len = np.asarray(text_len, dtype=np.int32).reshape(-1)
    rng = np.random.default_rng(seed)
    n_tokens = int(text_len.astype(np.int64).sum() + (grid_hw[:, 0].astype(np.int64) * grid_hw[:, 1]).sum())
    q, k, v = _draw_qkv(rng, n_tokens, heads, head_dim, dtype, scale)
    return Workload(name, grid_hw, text_len, heads, head_dim, dtype, q, k, v, seed)


@dataclass
class CfgBatch:
    """A packed classifier-free-guidance batch for one sampler step.

    Every image owns a conditional sample (its prompt, then its latent grid)
    and optionally an unconditional sample (unconditional prompt, same grid).
    ``z`` holds the images' latent tokens back to back (image order, each grid
    row-major); ``v`` holds a velocity for every token of the packed batch.
    """

    name: str
    grid_hw: np.ndarray  # int32 [n_seg, 2]
    text_len: np.ndarray  # int32 [n_seg]
    cond_seg: np.ndarray  # int32 [n_img]
    uncond_seg: np.ndarray  # int32 [n_img], -1: no unconditional sample
    channels: int
    dtype: str  # dtype of v: "bf16" or "f32"; z is always float32
    z: np.ndarray = field(repr=False)  # float32 [image_tokens, channels]
    v: np.ndarray = field(repr=False)  # float32 [tokens, channels], exactly representable in dtype
    seed: int = 0

    @property
    def n_seg(self) -> int:
        return int(self.grid_hw.shape[0])

    @property
    def n_img(self) -> int:
        return int(self.cond_seg.shape[0])

    @property
    def tokens(self) -> int:
        return int(self.v.shape[0])

    @property
    def image_tokens(self) -> int:
        return int(self.z.shape[0])


# Packed CFG batches: 1024x1024 images (64x64 latent grids, 128 latent channels
# per token), prompts uniform in [77, 256] tokens, unconditional prompt empty.
CFG_CONFIGS = {
    "cfg1024": dict(grids=[(64, 64)] * 8, uncond_text=0, channels=128, dtype="bf16", seed=6),
    "cfg_mixed": dict(grids=[(32, 128), (128, 32), (48, 84), (64, 64), (32, 32)], uncond_text=0, channels=128,
                      dtype="bf16", seed=7),
}


def make_cfg_batch(grids, cond_text=None, uncond_text=0, layout="interleaved", channels=128, dtype="bf16",
                   seed=0, guided=None, name="cfg", rng=None) -> CfgBatch:
    """Pack a CFG batch.

    grids: (h, w) per image. cond_text: prompt length per image, drawn uniformly
    in [77, 256] when None. uncond_text: prompt length of the unconditional
    samples (an int or one per image). guided: bool per image (default all);
    an unguided image has no unconditional sample. layout: "interleaved"
    (c0 u0 c1 u1 ...), "blocks" (all conditional samples, then all
    unconditional ones) or "shuffled" (a seeded permutation of the samples).
    Draw order: prompt lengths, permutation, then z ~ N(0, 1) and v ~ N(0, 1)
    as float32 (v rounded to bf16 for bf16 batches).
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    grids = [tuple(int(x) for x in g) for g in grids]
    n_img = len(grids)
    if cond_text is None:
        cond_text = rng.integers(77, 257, size=n_img).tolist()
    if np.isscalar(uncond_text):
        uncond_text = [int(uncond_text)] * n_img
    guided = [True] * n_img if guided is None else [bool(g) for g in guided]
    samples = []  # (image, is_cond)
    if layout == "blocks":
        samples = [(b, True) for b in range(n_img)] + [(b, False) for b in range(n_img) if guided[b]]
    else:
        for b in range(n_img):
            samples.append((b, True))
            if guided[b]:
                samples.append((b, False))
        if layout == "shuffled":
            samples = [samples[i] for i in rng.permutation(len(samples))]
        elif layout != "interleaved":
            raise ValueError(f"unknown layout {layout}")
    grid_hw = np.array([grids[b] for b, _ in samples], dtype=np.int32).reshape(-1, 2)
    text_len = np.array([cond_text[b] if c else uncond_text[b] for b, c in samples], dtype=np.int32)
    cond_seg = np.full(n_img, -1, dtype=np.int32)
    uncond_seg = np.full(n_img, -1, dtype=np.int32)
    for i, (b, c) in enumerate(samples):
        (cond_seg if c else uncond_seg)[b] = i
    image_tokens = sum(h * w for h, w in grids)
    tokens = int(text_len.astype(np.int64).sum() + (grid_hw[:, 0].astype(np.int64) * grid_hw[:, 1]).sum())
    z = rng.standard_normal((image_tokens, channels), dtype=np.float32)
    v = rng.standard_normal((tokens, channels), dtype=np.float32)
    if dtype == "bf16":
        v = bf16_bits_to_f32(f32_to_bf16_bits(v))
    return CfgBatch(name, grid_hw, text_len, cond_seg, uncond_seg, channels, dtype, z, v, seed)


def make_cfg_config(config: str, seed: int | None = None, layout="interleaved") -> CfgBatch:
    """The seeded CFG batch of a named config."""
    c = CFG_CONFIGS[config]
    seed = c["seed"] if seed is None else seed
    return make_cfg_batch(c["grids"], None, c["uncond_text"], layout, c["channels"], c["dtype"], seed,
                          name=config)


# Editing batches (tech report, NR-MMDiT editing paragraph): each sample is its
# instruction, then the source image latents, then the target latents, all on
# one grid; `frames` counts the images. The frame-aware RoPE split gives the
# row, column and frame blocks of a 128-channel head 48, 48 and 32 channels
# (the pages do not fix it; this is the proportion of the multimodal rotary
# layout of the vision-language text encoder the tech report names), 24/24/16
# for 64.
EDIT_SPLIT = {128: (48, 48, 32), 64: (24, 24, 16)}
EDIT_CONFIGS = {
    # One 1024x1024 edit: a 256-token instruction, a source and a target 64x64 grid.
    "edit1024": dict(grids=[(64, 64)], texts=[256], frames=[2], heads=24, head_dim=128, dtype="bf16", seed=8),
    # Three edits of mixed aspect, one or two source images, instructions of 77-256 tokens.
    "edit_mixed": dict(grids=[(32, 128), (64, 64), (48, 84)], texts="draw", frames=[2, 3, 2], heads=24,
                       head_dim=128, dtype="bf16", seed=9),
}


def make_edit(config=None, grids=None, texts=None, frames=None, heads=None, head_dim=None, dtype=None, seed=None,
              split=None, scale=1.0, name="edit") -> Workload:
    """An editing batch: a named config of EDIT_CONFIGS, or explicit segments.
    Draw order: prompt lengths (when drawn), then q, k, v as for make_workload."""
    if config is not None:
        c = EDIT_CONFIGS[config]
        grids, texts, frames = c["grids"], c["texts"], c["frames"]
        heads = c["heads"] if heads is None else heads
        head_dim = c["head_dim"] if head_dim is None else head_dim
        dtype = c["dtype"] if dtype is None else dtype
        seed = c["seed"] if seed is None else seed
        name = config
    rng = np.random.default_rng(0 if seed is None else seed)
    if isinstance(texts, str):
        texts = rng.integers(77, 257, size=len(grids)).tolist()
    grid_hw = np.asarray(grids, dtype=np.int32).reshape(-1, 2)
    text_len = np.asarray(texts, dtype=np.int32).reshape(-1)
    fr = np.asarray(frames, dtype=np.int32).reshape(-1)
    n_tokens = int(text_len.astype(np.int64).sum() + (fr.astype(np.int64) * grid_hw[:, 0] * grid_hw[:, 1]).sum())
    q, k, v = _draw_qkv(rng, n_tokens, heads, head_dim, dtype, scale)
    split = EDIT_SPLIT[head_dim] if split is None else tuple(split)
    return Workload(name, grid_hw, text_len, heads, head_dim, dtype, q, k, v, 0 if seed is None else seed, fr, split)


def make_qkv_inputs(grid_hw, text_len, hidden: int, heads: int, head_dim: int, frames=None, seed: int = 0):
    """Hidden states and synthetic modality-specific weights for the RMSNorm +
    packed QKV projection: x ~ N(0, 1) [T, hidden] (bf16 values), W_txt, W_img ~
    N(0, 1/hidden) [3 heads head_dim, hidden] (bf16 values), gains 1 + 0.1 N(0, 1)
    (float32). Draw order: x, W_txt, W_img, gamma_txt, gamma_img."""
    g = np.asarray(grid_hw, dtype=np.int64).reshape(-1, 2)
    t = np.asarray(text_len, dtype=np.int64).reshape(-1)
    f = np.ones_like(t) if frames is None else np.asarray(frames, dtype=np.int64).reshape(-1)
    T = int((t + f * g[:, 0] * g[:, 1]).sum())
    rng = np.random.default_rng(seed)
    rnd = lambda shape, s: bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * s))  # noqa: E731
    x = rnd((T, hidden), 1.0)
    w_txt = rnd((3 * heads * head_dim, hidden), 1.0 / np.sqrt(hidden))
    w_img = rnd((3 * heads * head_dim, hidden), 1.0 / np.sqrt(hidden))
    g_txt = (1.0 + 0.1 * rng.standard_normal(hidden)).astype(np.float32)
    g_img = (1.0 + 0.1 * rng.standard_normal(hidden)).astype(np.float32)
    return x, w_txt, w_img, g_txt, g_img
