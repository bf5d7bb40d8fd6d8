#!/usr/bin/env python3
"""Benchmark of packed joint text+image attention with 2D RoPE on one MI355X.

One step = one call of mf_attn_packed over the whole packed batch: metadata
check and tile table, 2D-RoPE prologue, per-sample flash attention. Inputs are
seeded synthetic tensors already resident in device memory; the library's own
metadata builder produces cu_seqlens before the timed region.

Prints one JSON line. `value` is packed joint-attention TFLOP/s, counting only
in-sample work: 4 * sum_i L_i^2 * head_dim * heads per step.

  python bench.py [--steps K] [--warmup W] [--config 1024sq|mixed|2048sq|train65k|tiny]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2.5e15, "f32": 157.3e12}  # dense MFMA bf16; fp32 vector ALU
HBM_PEAK = 8.0e12
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_1024sq_traffic.json")
KERNEL_SOURCES = [
    os.path.join(ROOT, "text_image_diffusion_varlen_amd", "csrc", name)
    for name in ("attn_fwd.hip", "mf_common.h", "mfma_util.h", "rope_math.h")
] + [os.path.join(ROOT, "text_image_diffusion_varlen_amd", "build.py")]  # compile flags
DESCRIPTIONS = {
    "tiny": "one 256x256 image (16x16 grid) + 32 prompt tokens, L=288, 2 heads x 64, fp32",
    "1024sq": "one 1024x1024 image (64x64 grid) + 256 prompt tokens, L=4352, 24 heads x 128, bf16",
    "mixed": "5 mixed-aspect images (32x128, 128x32, 48x84, 64x64, 32x32 grids) + prompts of 77-256 tokens, 24 heads x 128, bf16",
    "2048sq": "one 2048x2048 image (128x128 grid) + 256 prompt tokens, L=16640, 24 heads x 128, bf16",
    "train65k": "training-style packed block under a 65536-token budget, 24 heads x 128, bf16",
    "edit1024": "one 1024x1024 edit: 256-token instruction + source and target 64x64 grids (frames 0, 1), "
                "L=8448, frame-aware RoPE split 48/48/32, 24 heads x 128, bf16",
    "edit_mixed": "three edits (32x128 x2 frames, 64x64 x3, 48x84 x2) + instructions of 77-256 tokens, "
                  "frame-aware RoPE split 48/48/32, 24 heads x 128, bf16",
}


def kernel_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(config: str):
    """Measured HBM bytes per launch of the attention kernel, if the counters were
    taken on the current kernel source for this workload; else None."""
    if config != "1024sq" or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_sha():
        return None
    return rec.get("traffic_bytes")


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[a]), ctypes.c_void_p(self.ev[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def sample_lengths(w):
    f = 1 if w.frames is None else w.frames.astype("int64")
    return (w.text_len.astype("int64") + f * w.grid_hw[:, 0].astype("int64") * w.grid_hw[:, 1]).tolist()


def cpu_baseline(w, budget_s: float, gpu_out=None, gpu_meta=None):
    """The fp64 oracle (as it stands) on host cores, over as many whole heads of the
    same workload as fit in the time budget (at least one).

    After the timed loop, the oracle's outputs of those heads are compared with
    the GPU output of the same workload (`gpu_out`, [T][H][d] on the host) and
    the library's metadata (`gpu_meta` = (cu_seqlens, positions) on the host)
    with the oracle's packing: max / mean abs error, whether they are within
    the parity bars, and whether the metadata is bit-exact."""
    import numpy as np
    from oracle import attention, packing

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))
    lengths = sample_lengths(w)
    per_head = 4.0 * sum(L * L for L in lengths) * w.head_dim
    t0 = time.perf_counter()
    heads = 0
    outs = []
    while heads < w.heads:
        h = slice(heads, heads + 1)
        if w.frames is None:
            o = attention.joint_attention(w.q[:, h], w.k[:, h], w.v[:, h], w.grid_hw, w.text_len)
        else:
            o = attention.joint_attention_3d(w.q[:, h], w.k[:, h], w.v[:, h], w.grid_hw, w.text_len, w.frames,
                                             w.rope_split)
        outs.append(o)
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    res = {
        "value": per_head * heads / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{heads} of {w.heads} heads of the same workload (all rows, fp64 numpy), {dt:.1f} s",
    }
    if gpu_out is not None:
        err = np.abs(gpu_out[:, :heads].astype(np.float64) - np.concatenate(outs, axis=1))
        bars = (2e-2, 2e-3) if w.dtype == "bf16" else (1e-5, 1e-5)
        res["max_abs_err_vs_gpu"] = float(err.max())
        res["mean_abs_err_vs_gpu"] = float(err.mean())
        res["within_parity_bars"] = bool(err.max() <= bars[0] and err.mean() <= bars[1])
    if gpu_meta is not None:
        cu, pos = gpu_meta
        if w.frames is None:
            ref_pos, _ = packing.token_positions(w.grid_hw, w.text_len)
        else:
            ref_pos, _ = packing.token_positions_3d(w.grid_hw, w.text_len, w.frames)
        ref_cu = packing.cu_seqlens(w.grid_hw, w.text_len, w.frames)
        res["metadata_bit_exact"] = bool(np.array_equal(cu, ref_cu) and np.array_equal(pos, ref_pos))
    return res


def sampler_bench(steps: int, warmup: int):
    """Guided Euler step over the packed CFG batch of eight 1024x1024 images.

    Back-to-back steps rotate over enough copies of (z, v) to span three times
    the 256 MB last-level cache, so every step reads z and v from HBM; one event
    pair brackets all timed steps. The steps are timed as a captured HIP graph
    (launch cost off the host) and, for reference, as eager calls. HBM GB/s is
    computed from the algorithmic bytes (read z, v_c, v_u; write z)."""
    import torch
    from text_image_diffusion_varlen_amd import binding, workloads

    b = workloads.make_cfg_config("cfg1024")
    grid = torch.from_numpy(b.grid_hw).cuda()
    text = torch.from_numpy(b.text_len).cuda()
    cu, _, _ = binding.build_metadata(grid, text, b.tokens)
    cs = torch.from_numpy(b.cond_seg).cuda()
    us = torch.from_numpy(b.uncond_seg).cuda()
    set_bytes = b.z.nbytes + b.v.size * 2
    n_sets = max(2, -(-3 * 256 * 2**20 // set_bytes))
    z0 = torch.from_numpy(b.z).cuda()
    v0 = torch.from_numpy(b.v).to(torch.bfloat16).cuda()
    sets = [(z0.clone(), v0.clone()) for _ in range(n_sets)]
    step = lambda z, v: binding.rf_cfg_euler_step(z, v, cu, grid, text, cs, us, 5.0, 0.25)  # noqa: E731
    for i in range(max(warmup, n_sets)):
        step(*sets[i % n_sets])
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Eager: one library call per step from Python (host launch cost included).
    start.record()
    for i in range(steps):
        step(*sets[i % n_sets])
    stop.record()
    torch.cuda.synchronize()
    eager = start.elapsed_time(stop) / 1e3 / steps
    # Graph: one pass over every buffer set captured once and replayed, as a
    # sampler loop would run it.
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for zv in sets:
            step(*zv)
    reps = max(1, steps // n_sets)
    g.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    sec = start.elapsed_time(stop) / 1e3 / (reps * n_sets)
    if binding.get_device_error() != binding.MF_OK:
        raise RuntimeError(binding.last_error())
    nbytes = b.image_tokens * b.channels * (4 + 4 + 2 + 2)
    # Context: torch.add of two fp32 tensors of z's size into a third moves the
    # same bytes (reads 2 x 4 B, writes 4 B per element), timed the same way.
    del sets, g
    n = b.image_tokens * b.channels
    adds = [tuple(torch.empty(n, dtype=torch.float32, device="cuda").normal_() for _ in range(3))
            for _ in range(n_sets)]
    for x, y, o in adds:
        torch.add(x, y, out=o)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, y, o in adds:
            torch.add(x, y, out=o)
    g.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    add_sec = start.elapsed_time(stop) / 1e3 / (reps * n_sets)
    del adds, g
    return {
        "workload": "cfg1024: 8 images of 64x64 latent tokens x 128 channels, conditional + empty-prompt "
                    "unconditional samples interleaved, bf16 velocities, fp32 latents",
        "us_per_step": round(sec * 1e6, 2),
        "us_per_step_eager": round(eager * 1e6, 2),
        "gbps": round(nbytes / sec / 1e9, 1),
        "frac_hbm": round(nbytes / sec / HBM_PEAK, 4),
        "torch_add_same_bytes_us": round(add_sec * 1e6, 2),
        "algorithmic_bytes": nbytes,
        "buffer_sets": n_sets,
    }


def backward_bench(w, q, k, v, cu, grid, text, steps: int, warmup: int, frames=None):
    """Packed backward on the same batch: one step = mf_attn_packed_bwd (metadata,
    prologue, dK/dV kernel, dQ kernel) with the forward's out and LSE resident.
    TFLOP/s count the algorithmic 10 * sum_i L_i^2 * d * H (the five products of
    the backward; the kernels' recomputation of S and dP is not counted)."""
    import torch
    from text_image_diffusion_varlen_amd import binding

    if frames is None:
        out, lse = binding.attn_packed_lse(q, k, v, cu, grid, text)
    else:
        out, lse = binding.attn_packed_3d(q, k, v, cu, grid, text, frames, w.rope_split, lse=True)
    gen = torch.Generator(device="cuda").manual_seed(5)
    d_out = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(q.dtype)
    grads = tuple(torch.empty_like(q) for _ in range(3))

    def bwd():
        if frames is None:
            binding.attn_packed_bwd(q, k, v, out, d_out, lse, cu, grid, text, grads=grads)
        else:
            binding.attn_packed_3d_bwd(q, k, v, out, d_out, lse, cu, grid, text, frames, w.rope_split, grads=grads)
    for _ in range(warmup):
        bwd()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        bwd()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    lengths = sample_lengths(w)
    per = sum(L * L for L in lengths) * w.head_dim * w.heads
    if frames is not None:
        if binding.get_device_error() != binding.MF_OK:
            raise RuntimeError(binding.last_error())
        return {"tflops": round(10.0 * per / (ms / 1e3) / 1e12, 2), "ms_per_step": round(ms, 4),
                "flop_per_step": 10.0 * per}
    ev = HipEvents(4 * steps)
    for st in range(steps):
        binding.attn_packed_bwd_profiled(q, k, v, out, d_out, lse, cu, grid, text, ev.ev[4 * st:4 * st + 4],
                                         grads=grads)
    torch.cuda.synchronize()
    if binding.get_device_error() != binding.MF_OK:
        raise RuntimeError(binding.last_error())
    stage = {"meta_pack": 0.0, "dkdv": 0.0, "dq": 0.0}
    for st in range(steps):
        b = 4 * st
        stage["meta_pack"] += ev.elapsed_ms(b, b + 1) / steps
        stage["dkdv"] += ev.elapsed_ms(b + 1, b + 2) / steps
        stage["dq"] += ev.elapsed_ms(b + 2, b + 3) / steps
    ev.close()
    flops = 10.0 * per
    # MFMA work the two kernels execute (S and dP are recomputed by the dQ kernel):
    # dK/dV kernel S, dP, dV, dK = 8 L^2 d H; dQ kernel S, dP, dQ = 6 L^2 d H
    kv_flops, q_flops = 8.0 * per, 6.0 * per
    return {
        "tflops": round(flops / (ms / 1e3) / 1e12, 2),
        "ms_per_step": round(ms, 4),
        "flop_per_step": flops,
        "stages_ms": {k2: round(v2, 4) for k2, v2 in stage.items()},
        "dkdv_executed_tflops": round(kv_flops / (stage["dkdv"] / 1e3) / 1e12, 1),
        "dq_executed_tflops": round(q_flops / (stage["dq"] / 1e3) / 1e12, 1),
        "pct_mfma_peak_executed": round(100.0 * (kv_flops + q_flops) / ((stage["dkdv"] + stage["dq"]) / 1e3) / PEAK["bf16"], 2),
    }


def qkv_bench(w, grid, text, cu, steps: int, warmup: int, frames=None):
    """Modality-specific RMSNorm + packed QKV projection feeding the same batch:
    hidden = heads * head_dim (3072 for 24 x 128), synthetic weights. TFLOP/s
    count 2 * T * hidden * 3 * heads * head_dim. For context, torch.matmul
    (hipBLASLt) of one [T, hidden] x [hidden, 3 heads head_dim] bf16 product of
    the same size is timed too (no normalization, one weight for all tokens)."""
    import torch
    from text_image_diffusion_varlen_amd import binding, workloads

    hidden = w.heads * w.head_dim
    x, wt, wi, gt, gi = workloads.make_qkv_inputs(w.grid_hw, w.text_len, hidden, w.heads, w.head_dim, w.frames,
                                                  seed=11)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()  # noqa: E731
    xd = bf(x)
    wf = binding.qkv_fold_weights(bf(wt), bf(wi), torch.from_numpy(gt).cuda(), torch.from_numpy(gi).cuda(),
                                  w.heads, w.head_dim)
    out = tuple(torch.empty((w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    for _ in range(warmup):
        binding.qkv_rmsnorm(xd, wf, cu, grid, text, w.heads, w.head_dim, frames=frames, out=out)
    torch.cuda.synchronize()
    ev = HipEvents(3 * steps)
    for st in range(steps):
        binding.qkv_rmsnorm(xd, wf, cu, grid, text, w.heads, w.head_dim, frames=frames, out=out,
                            events=ev.ev[3 * st:3 * st + 3])
    torch.cuda.synchronize()
    if binding.get_device_error() != binding.MF_OK:
        raise RuntimeError(binding.last_error())
    stats = sum(ev.elapsed_ms(3 * st, 3 * st + 1) for st in range(steps)) / steps
    gemm = sum(ev.elapsed_ms(3 * st + 1, 3 * st + 2) for st in range(steps)) / steps
    ev.close()
    flops = 2.0 * w.tokens * hidden * 3 * w.heads * w.head_dim
    wplain = bf(wt).t().contiguous()
    y = torch.matmul(xd, wplain)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        torch.matmul(xd, wplain, out=y)
    stop.record()
    torch.cuda.synchronize()
    mm = start.elapsed_time(stop) / steps
    return {
        "tflops": round(flops / ((stats + gemm) / 1e3) / 1e12, 1),
        "us_per_call": round((stats + gemm) * 1e3, 2),
        "stages_us": {"route_rms": round(stats * 1e3, 2), "gemm": round(gemm * 1e3, 2)},
        "gemm_tflops": round(flops / (gemm / 1e3) / 1e12, 1),
        "gemm_frac_mfma_peak": round(flops / (gemm / 1e3) / PEAK["bf16"], 4),
        "flop_per_call": flops,
        "hidden": hidden,
        "torch_matmul_same_size_tflops": round(flops / (mm / 1e3) / 1e12, 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="1024sq", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sampler", action="store_true", help="skip the packed CFG Euler-step measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the packed backward measurement")
    ap.add_argument("--no-qkv", action="store_true", help="skip the RMSNorm + QKV projection measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB (HBM-counter calibration for profiling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(a packed batch would shard by whole samples, one process per GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    from text_image_diffusion_varlen_amd import binding, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n,
                          "dispatches": max(args.steps, 1)}), flush=True)
        return
    edit = args.config in workloads.EDIT_CONFIGS
    w = workloads.make_edit(args.config, seed=args.seed) if edit else workloads.make_workload(args.config, seed=args.seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dt).cuda() for x in (w.q, w.k, w.v))
    grid = torch.from_numpy(w.grid_hw).cuda()
    text = torch.from_numpy(w.text_len).cuda()
    if edit:
        frames = torch.from_numpy(w.frames).cuda()
        cu, pos, _ = binding.build_metadata_3d(grid, text, frames, w.tokens)
    else:
        cu, pos, _ = binding.build_metadata(grid, text, w.tokens)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    if binding.get_device_error() != binding.MF_OK:
        raise RuntimeError(binding.last_error())

    lengths = sample_lengths(w)
    flops = 4.0 * sum(L * L for L in lengths) * w.head_dim * w.heads
    elem = 2 if w.dtype == "bf16" else 4
    qkvo_bytes = 4.0 * w.tokens * w.heads * w.head_dim * elem

    if edit:
        def step():
            binding.attn_packed_3d(q, k, v, cu, grid, text, frames, w.rope_split, out=out)
    else:
        def step():
            binding.attn_packed(q, k, v, cu, grid, text, out=out)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps, torch events on the stream the library launches on.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    if binding.get_device_error() != binding.MF_OK:
        raise RuntimeError(binding.last_error())

    # Per-kernel durations: the same calls with HIP events between the three
    # kernels (2D path; the frame-aware batches report the whole step).
    if edit:
        stage = {"meta": 0.0, "rope_pack": 0.0, "attn": ms}
    else:
        ev = HipEvents(4 * args.steps)
        for s in range(args.steps):
            binding.attn_packed_profiled(q, k, v, cu, grid, text, ev.ev[4 * s : 4 * s + 4], out=out)
        torch.cuda.synchronize()
        stage = {"meta": 0.0, "rope_pack": 0.0, "attn": 0.0}
        attn_each = []
        for s in range(args.steps):
            b = 4 * s
            stage["meta"] += ev.elapsed_ms(b, b + 1) / args.steps
            stage["rope_pack"] += ev.elapsed_ms(b + 1, b + 2) / args.steps
            attn_each.append(ev.elapsed_ms(b + 2, b + 3))
        stage["attn"] = sum(attn_each) / args.steps
        # The same calls with the 256 MB MALL flushed before each (a 512 MB
        # buffer written in between): the RoPE prologue then reads k and v from HBM.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        pack_cold = []
        for s in range(args.steps):
            flush.fill_(s & 255)
            binding.attn_packed_profiled(q, k, v, cu, grid, text, ev.ev[4 * s : 4 * s + 4], out=out)
        torch.cuda.synchronize()
        for s in range(args.steps):
            pack_cold.append(ev.elapsed_ms(4 * s + 1, 4 * s + 2))
        del flush
        ev.close()

    # The forward output and metadata of this workload, for the oracle comparison
    # in the CPU baseline (the last call above ran the same inputs).
    gpu_out = gpu_meta = None
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        gpu_out = out.float().cpu().numpy()
        gpu_meta = (cu.cpu().numpy(), pos.cpu().numpy())

    attn_s = stage["attn"] / 1e3
    achieved = flops / attn_s
    # prologue: bf16 reads k, v and writes K~, V~ (queries are rotated inside the attention kernel);
    # f32 also reads q and writes Q~
    rope_bytes = (4.0 if w.dtype == "bf16" else 6.0) * w.tokens * w.heads * w.head_dim * elem
    result = {
        "metric": "packed joint-attn TFLOP/s (bf16, 2D RoPE) + % of MFMA peak; tokens/s",
        "value": round(flops / (ms / 1e3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {DESCRIPTIONS[args.config]}",
            "tokens": w.tokens,
            "samples": w.n_seg,
            "heads": w.heads,
            "head_dim": w.head_dim,
            "seed": w.seed,
            "flop_per_step": flops,
        },
        "pct_mfma_peak": round(100.0 * flops / (ms / 1e3) / PEAK[w.dtype], 2),
        "tokens_per_s": round(w.tokens / (ms / 1e3), 1),
        "stages_ms": {k2: round(v2, 4) for k2, v2 in stage.items()},
        "attn_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(attn_each, [10, 50, 90])] if not edit else None,
        "rope_pack_gbps": round(rope_bytes / (stage["rope_pack"] / 1e3) / 1e9, 1) if not edit else None,
        "rope_pack_gbps_cold_mall": round(rope_bytes / (float(np.median(pack_cold)) / 1e3) / 1e9, 1) if not edit else None,
        "roofline": {
            "kernel": f"attn_fwd_{w.dtype}_kernel<{w.head_dim}, {'true' if edit else 'false'}>"
                      + (" (whole step: no per-kernel events on the frame-aware path)" if edit else ""),
            "bound": "mfma" if w.dtype == "bf16" else "alu",
            "achieved": round(achieved / 1e12, 2),
            "peak": PEAK[w.dtype] / 1e12,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK[w.dtype], 4),
            "traffic": stored_traffic(args.config),
            "algorithmic_bytes": qkvo_bytes,
        },
    }
    if w.dtype == "bf16" and not args.no_backward:
        result["backward"] = backward_bench(w, q, k, v, cu, grid, text, args.steps, args.warmup,
                                            frames if edit else None)
    if w.dtype == "bf16" and not args.no_qkv:
        result["qkv_rmsnorm"] = qkv_bench(w, grid, text, cu, args.steps, args.warmup, frames if edit else None)
    if not args.no_sampler:
        result["cfg_euler_step"] = sampler_bench(args.steps, args.warmup)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, gpu_out=gpu_out, gpu_meta=gpu_meta)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
