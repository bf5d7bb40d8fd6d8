"""ctypes binding of libmfattn.so (argument marshalling only).

Every function here checks tensor properties, passes raw device pointers and
the current HIP stream to the C ABI declared in include/mf_attn.h, and raises
MFError on a negative status. All arithmetic runs in the library's kernels;
there is no fallback path: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmfattn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "mf_attn.h")

MF_OK = 0
MF_ERR_INVALID_ARG = -1
MF_ERR_METADATA = -2
MF_ERR_UNSUPPORTED = -3
MF_ERR_HIP = -4
MF_ERR_OOM = -5
MF_BF16 = 0
MF_F32 = 1
ROPE_THETA = 10000.0

_DTYPES = {torch.bfloat16: MF_BF16, torch.float32: MF_F32}
_lib = None


class MFError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"mfattn error {code}: {message}")
        self.code = code


class MfTensor(ctypes.Structure):
    """mf_tensor: strided tensor descriptor of the C ABI."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("stride_token", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


def _declare(lib):
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "mf_version": ([], ctypes.c_int),
        "mf_last_error": ([], ctypes.c_char_p),
        "mf_attn_packed": ([P, P, P, P, P, P, P, I32, I64, I32, I32, I32, P], ctypes.c_int),
        "mf_attn_packed_profiled": ([P, P, P, P, P, P, P, I32, I64, I32, I32, I32, P, P], ctypes.c_int),
        "mf_workspace_bytes": ([I64, I32, I32, I32, I32], SZ),
        "mf_attn_packed_ws": ([P, P, P, P, P, P, P, I32, I64, I32, I32, I32, P, SZ, P], ctypes.c_int),
        "mf_attn_packed_noalloc": ([P, P, P, P, P, P, P, I32, I64, I32, I32, I32, P], ctypes.c_int),
        "mf_attn_packed_strided": ([P, P, P, P, P, P, I32, P, P], ctypes.c_int),
        "mf_attn_packed_lse": ([P, P, P, P, P, P, P, P, I32, I64, I32, I32, I32, P], ctypes.c_int),
        "mf_attn_packed_bwd": ([P] * 12 + [I32, I64, I32, I32, I32, P], ctypes.c_int),
        "mf_attn_packed_bwd_profiled": ([P] * 12 + [I32, I64, I32, I32, I32, P, P], ctypes.c_int),
        "mf_bwd_workspace_bytes": ([I64, I32, I32, I32], SZ),
        "mf_attn_packed_3d": ([P] * 7 + [I32, I32, I32, P, P, I32, I64, I32, I32, I32, P], ctypes.c_int),
        "mf_attn_packed_3d_bwd": ([P] * 10 + [I32, I32, I32, P, P, P, I32, I64, I32, I32, I32, P], ctypes.c_int),
        "mf_build_metadata_3d": ([I32, P, P, P, P, P, P, I64, P], ctypes.c_int),
        "mf_rope_3d": ([P, P, P, I64, I32, I32, I32, F, I32, I32, I32, P], ctypes.c_int),
        "mf_build_metadata": ([I32, P, P, P, P, P, I64, P], ctypes.c_int),
        "mf_rope_2d": ([P, P, P, I64, I32, I32, I32, F, P], ctypes.c_int),
        "mf_rf_cfg_euler_step": ([P, P, P, P, P, I32, I64, P, P, I32, I64, I32, I32, F, F, P], ctypes.c_int),
        "mf_qkv_fold_weights": ([P, P, P, P, I32, I32, I32, P, P], ctypes.c_int),
        "mf_qkv_rmsnorm": ([P] * 6 + [I32, I64, I32, I32, I32, F, P, P, P, P], ctypes.c_int),
        "mf_qkv_rmsnorm_profiled": ([P] * 6 + [I32, I64, I32, I32, I32, F, P, P, P, P, P], ctypes.c_int),
        "mf_pack_joint": ([I32, P, P, P, P, P, P, P, I32, I64, I64, I32, I32, I32, P], ctypes.c_int),
        "mf_unpack_joint": ([I32, P, P, P, P, P, P, P, I32, I64, I64, I32, I32, I32, P], ctypes.c_int),
        "mf_get_device_error": ([P], ctypes.c_int),
        "mf_get_workspace_error": ([P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m text_image_diffusion_varlen_amd.build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def header_functions():
    """Names of the functions declared in include/mf_attn.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(mf_\w+)\(", text, re.M)))


def _check(rc: int):
    if rc != MF_OK:
        raise MFError(rc, lib().mf_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, ndim=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def version() -> int:
    return lib().mf_version()


def workspace_bytes(total_tokens: int, heads: int, head_dim: int, dtype: torch.dtype, n_seg: int) -> int:
    return int(lib().mf_workspace_bytes(total_tokens, heads, head_dim, _DTYPES[dtype], n_seg))


def _attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, ndim=3)
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype in {bfloat16, float32}")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same [tokens, heads, head_dim] shape")
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(grid_hw, "grid_hw", torch.int32, 2)
    _need(text_len, "text_len", torch.int32, 1)
    n = grid_hw.shape[0]
    if grid_hw.shape[1] != 2 or text_len.shape[0] != n or cu_seqlens.shape[0] != n + 1:
        raise ValueError("metadata shapes must be grid_hw [n,2], text_len [n], cu_seqlens [n+1]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, 3)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    T, H, D = q.shape
    return out, n, T, H, D


def attn_packed(q, k, v, cu_seqlens, grid_hw, text_len, out=None, stream=None):
    """Packed joint attention with 2D RoPE (mf_attn_packed). Returns out."""
    out, n, T, H, D = _attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out)
    _check(lib().mf_attn_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len),
                                _ptr(out), n, T, H, D, _DTYPES[q.dtype], _stream(stream)))
    return out


def attn_packed_profiled(q, k, v, cu_seqlens, grid_hw, text_len, events, out=None, stream=None):
    """mf_attn_packed recording four hipEvent_t handles (ints) between its kernels."""
    out, n, T, H, D = _attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out)
    arr = (ctypes.c_void_p * 4)(*events)
    _check(lib().mf_attn_packed_profiled(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(grid_hw),
                                         _ptr(text_len), _ptr(out), n, T, H, D, _DTYPES[q.dtype],
                                         ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))
    return out


def attn_packed_ws(q, k, v, cu_seqlens, grid_hw, text_len, workspace, out=None, stream=None):
    """mf_attn_packed_ws with a caller-owned uint8 device workspace."""
    out, n, T, H, D = _attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out)
    _need(workspace, "workspace", torch.uint8, 1)
    _check(lib().mf_attn_packed_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len),
                                   _ptr(out), n, T, H, D, _DTYPES[q.dtype], _ptr(workspace),
                                   workspace.numel(), _stream(stream)))
    return out


def attn_packed_noalloc(q, k, v, cu_seqlens, grid_hw, text_len, out, stream=None):
    """mf_attn_packed_noalloc: the forward on the library's fixed static scratch.
    `out` must be given (this call allocates nothing). Returns out."""
    out, n, T, H, D = _attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out)
    _check(lib().mf_attn_packed_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(grid_hw),
                                        _ptr(text_len), _ptr(out), n, T, H, D, _DTYPES[q.dtype], _stream(stream)))
    return out


def _descriptor(t, name):
    """mf_tensor of a [tokens, heads, head_dim] view whose channels are contiguous."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 3:
        raise ValueError(f"{name} must be a 3-dim device tensor")
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name} must be bfloat16 or float32")
    if t.stride(2) != 1:
        raise ValueError(f"{name} must have contiguous channels")
    T, H, D = t.shape
    return MfTensor(t.data_ptr(), _DTYPES[t.dtype], T, H, D, t.stride(0), t.stride(1))


def attn_packed_strided(q, k, v, cu_seqlens, grid_hw, text_len, out, stream=None):
    """mf_attn_packed_strided: the forward on strided [T, H, d] views (channels
    contiguous), e.g. slices of one fused QKV buffer. Returns out."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(grid_hw, "grid_hw", torch.int32, 2)
    _need(text_len, "text_len", torch.int32, 1)
    d = [_descriptor(t, name) for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out"))]
    ptr = lambda x: ctypes.cast(ctypes.pointer(x), ctypes.c_void_p)  # noqa: E731
    _check(lib().mf_attn_packed_strided(ptr(d[0]), ptr(d[1]), ptr(d[2]), _ptr(cu_seqlens), _ptr(grid_hw),
                                        _ptr(text_len), grid_hw.shape[0], ptr(d[3]), _stream(stream)))
    return out


def attn_packed_lse(q, k, v, cu_seqlens, grid_hw, text_len, out=None, lse=None, stream=None):
    """Forward that also returns the row log-sum-exp (mf_attn_packed_lse): (out, lse [H, T] float32)."""
    out, n, T, H, D = _attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, 2)
    if lse.shape != (H, T):
        raise ValueError("lse must be [heads, tokens]")
    _check(lib().mf_attn_packed_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len),
                                    _ptr(out), _ptr(lse), n, T, H, D, _DTYPES[q.dtype], _stream(stream)))
    return out, lse


def _bwd_args(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, grads):
    _, n, T, H, D = _attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out)
    _need(d_out, "d_out", q.dtype, 3)
    if d_out.shape != q.shape:
        raise ValueError("d_out must have the shape of q")
    _need(lse, "lse", torch.float32, 2)
    if lse.shape != (H, T):
        raise ValueError("lse must be [heads, tokens]")
    if grads is None:
        grads = tuple(torch.empty_like(q) for _ in range(3))
    for name, g in zip(("dq", "dk", "dv"), grads):
        _need(g, name, q.dtype, 3)
        if g.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    return grads, n, T, H, D


def attn_packed_bwd(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, grads=None, stream=None):
    """Packed backward (mf_attn_packed_bwd). Returns (dq, dk, dv)."""
    (dq, dk, dv), n, T, H, D = _bwd_args(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, grads)
    _check(lib().mf_attn_packed_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(d_out), _ptr(lse),
                                    _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len), _ptr(dq), _ptr(dk),
                                    _ptr(dv), n, T, H, D, _DTYPES[q.dtype], _stream(stream)))
    return dq, dk, dv


def attn_packed_bwd_profiled(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, events, grads=None,
                             stream=None):
    """mf_attn_packed_bwd recording four hipEvent_t handles (ints) between its kernels."""
    (dq, dk, dv), n, T, H, D = _bwd_args(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, grads)
    arr = (ctypes.c_void_p * 4)(*events)
    _check(lib().mf_attn_packed_bwd_profiled(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(d_out), _ptr(lse),
                                             _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len), _ptr(dq),
                                             _ptr(dk), _ptr(dv), n, T, H, D, _DTYPES[q.dtype],
                                             ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))
    return dq, dk, dv


def _split(split, head_dim):
    split = tuple(int(x) for x in split)
    if len(split) != 3:
        raise ValueError("split must have three entries (row, col, frame)")
    return split


def attn_packed_3d(q, k, v, cu_seqlens, grid_hw, text_len, frames, split, out=None, lse=False, stream=None):
    """Frame-aware packed attention (mf_attn_packed_3d). Returns out, or (out, lse) when lse is True
    or a [H, T] float32 tensor."""
    out, n, T, H, D = _attn_args(q, k, v, cu_seqlens, grid_hw, text_len, out)
    _need(frames, "frames", torch.int32, 1)
    if frames.shape[0] != n:
        raise ValueError("frames must be [n]")
    sr, sc, sf = _split(split, D)
    want = lse is not False and lse is not None
    if lse is True:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    if want:
        _need(lse, "lse", torch.float32, 2)
        if lse.shape != (H, T):
            raise ValueError("lse must be [heads, tokens]")
    _check(lib().mf_attn_packed_3d(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len),
                                   _ptr(frames), sr, sc, sf, _ptr(out), _ptr(lse) if want else None, n, T, H, D,
                                   _DTYPES[q.dtype], _stream(stream)))
    return (out, lse) if want else out


def attn_packed_3d_bwd(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, frames, split, grads=None,
                       stream=None):
    """Backward of the frame-aware attention (mf_attn_packed_3d_bwd). Returns (dq, dk, dv)."""
    (dq, dk, dv), n, T, H, D = _bwd_args(q, k, v, out, d_out, lse, cu_seqlens, grid_hw, text_len, grads)
    _need(frames, "frames", torch.int32, 1)
    sr, sc, sf = _split(split, D)
    _check(lib().mf_attn_packed_3d_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(d_out), _ptr(lse),
                                       _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len), _ptr(frames), sr, sc, sf,
                                       _ptr(dq), _ptr(dk), _ptr(dv), n, T, H, D, _DTYPES[q.dtype],
                                       _stream(stream)))
    return dq, dk, dv


def build_metadata_3d(grid_hw, text_len, frames, total_tokens: int, stream=None):
    """(cu_seqlens [n+1], pos [T,3], seg_id [T]) for editing samples (mf_build_metadata_3d)."""
    _need(grid_hw, "grid_hw", torch.int32, 2)
    _need(text_len, "text_len", torch.int32, 1)
    _need(frames, "frames", torch.int32, 1)
    n = grid_hw.shape[0]
    dev = grid_hw.device
    cu = torch.empty(n + 1, dtype=torch.int32, device=dev)
    pos = torch.empty((total_tokens, 3), dtype=torch.int32, device=dev)
    seg = torch.empty(total_tokens, dtype=torch.int32, device=dev)
    _check(lib().mf_build_metadata_3d(n, _ptr(grid_hw), _ptr(text_len), _ptr(frames), _ptr(cu), _ptr(pos),
                                      _ptr(seg), total_tokens, _stream(stream)))
    return cu, pos, seg


def rope_3d(x, pos, split, theta: float = ROPE_THETA, out=None, stream=None):
    """Frame-aware RoPE of x [T, H, d] at pos [T, 3] (mf_rope_3d). Returns out."""
    _need(x, "x", ndim=3)
    _need(pos, "pos", torch.int32, 2)
    if x.dtype not in _DTYPES:
        raise ValueError("x must be bfloat16 or float32")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, 3)
    T, H, D = x.shape
    if pos.shape != (T, 3) or out.shape != x.shape:
        raise ValueError("shape mismatch")
    sr, sc, sf = _split(split, D)
    _check(lib().mf_rope_3d(_ptr(x), _ptr(out), _ptr(pos), T, H, D, _DTYPES[x.dtype], float(theta), sr, sc, sf,
                            _stream(stream)))
    return out


def build_metadata(grid_hw, text_len, total_tokens: int, stream=None):
    """(cu_seqlens [n+1], pos [T,2], seg_id [T]) int32 device tensors (mf_build_metadata)."""
    _need(grid_hw, "grid_hw", torch.int32, 2)
    _need(text_len, "text_len", torch.int32, 1)
    n = grid_hw.shape[0]
    dev = grid_hw.device
    cu = torch.empty(n + 1, dtype=torch.int32, device=dev)
    pos = torch.empty((total_tokens, 2), dtype=torch.int32, device=dev)
    seg = torch.empty(total_tokens, dtype=torch.int32, device=dev)
    _check(lib().mf_build_metadata(n, _ptr(grid_hw), _ptr(text_len), _ptr(cu), _ptr(pos), _ptr(seg),
                                   total_tokens, _stream(stream)))
    return cu, pos, seg


def rope_2d(x, pos, theta: float = ROPE_THETA, out=None, stream=None):
    """2D RoPE of x [T, H, d] at pos [T, 2] (mf_rope_2d). Returns out."""
    _need(x, "x", ndim=3)
    _need(pos, "pos", torch.int32, 2)
    if x.dtype not in _DTYPES:
        raise ValueError("x must be bfloat16 or float32")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, 3)
    T, H, D = x.shape
    if pos.shape[0] != T or out.shape != x.shape:
        raise ValueError("shape mismatch")
    _check(lib().mf_rope_2d(_ptr(x), _ptr(out), _ptr(pos), T, H, D, _DTYPES[x.dtype], float(theta),
                            _stream(stream)))
    return out


def rf_cfg_euler_step(z, v, cu_seqlens, grid_hw, text_len, cond_seg, uncond_seg, guidance: float, dt: float,
                      stream=None):
    """In-place guided Euler step z += dt * (v_u + guidance * (v_c - v_u)) (mf_rf_cfg_euler_step).

    z [image_tokens, C] float32; v [total_tokens, C] bfloat16/float32; cond_seg,
    uncond_seg [n_img] int32 sample indices (uncond -1: no guidance). Returns z.
    """
    _need(z, "z", torch.float32, 2)
    _need(v, "v", ndim=2)
    if v.dtype not in _DTYPES:
        raise ValueError("v must be bfloat16 or float32")
    if v.shape[1] != z.shape[1]:
        raise ValueError("z and v must have the same channel count")
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(grid_hw, "grid_hw", torch.int32, 2)
    _need(text_len, "text_len", torch.int32, 1)
    _need(cond_seg, "cond_seg", torch.int32, 1)
    _need(uncond_seg, "uncond_seg", torch.int32, 1)
    n = grid_hw.shape[0]
    if grid_hw.shape[1] != 2 or text_len.shape[0] != n or cu_seqlens.shape[0] != n + 1:
        raise ValueError("metadata shapes must be grid_hw [n,2], text_len [n], cu_seqlens [n+1]")
    if uncond_seg.shape != cond_seg.shape:
        raise ValueError("cond_seg and uncond_seg must have the same length")
    _check(lib().mf_rf_cfg_euler_step(_ptr(z), _ptr(v), _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len), n,
                                      v.shape[0], _ptr(cond_seg), _ptr(uncond_seg), cond_seg.shape[0],
                                      z.shape[0], z.shape[1], _DTYPES[v.dtype], float(guidance), float(dt),
                                      _stream(stream)))
    return z


def qkv_fold_weights(w_txt, w_img, gamma_txt, gamma_img, heads: int, head_dim: int, out=None, stream=None):
    """Gains folded into the packed QKV weights (mf_qkv_fold_weights): [2, 3HD, hidden] bf16."""
    for name, t in (("w_txt", w_txt), ("w_img", w_img)):
        _need(t, name, torch.bfloat16, 2)
    for name, t in (("gamma_txt", gamma_txt), ("gamma_img", gamma_img)):
        _need(t, name, torch.float32, 1)
    n_out, hidden = w_txt.shape
    if w_img.shape != w_txt.shape or n_out != 3 * heads * head_dim or gamma_txt.shape[0] != hidden \
            or gamma_img.shape[0] != hidden:
        raise ValueError("weights must be [3*heads*head_dim, hidden] and gains [hidden]")
    if out is None:
        out = torch.empty((2, n_out, hidden), dtype=torch.bfloat16, device=w_txt.device)
    _need(out, "out", torch.bfloat16, 3)
    _check(lib().mf_qkv_fold_weights(_ptr(w_txt), _ptr(w_img), _ptr(gamma_txt), _ptr(gamma_img), hidden, heads,
                                     head_dim, _ptr(out), _stream(stream)))
    return out


def qkv_rmsnorm(x, w_folded, cu_seqlens, grid_hw, text_len, heads: int, head_dim: int, frames=None, eps: float = 1e-6,
                out=None, events=None, stream=None):
    """Modality-specific RMSNorm + packed QKV projection (mf_qkv_rmsnorm). Returns (q, k, v) [T, H, d]."""
    _need(x, "x", torch.bfloat16, 2)
    _need(w_folded, "w_folded", torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(grid_hw, "grid_hw", torch.int32, 2)
    _need(text_len, "text_len", torch.int32, 1)
    T, hidden = x.shape
    n = grid_hw.shape[0]
    if w_folded.shape != (2, 3 * heads * head_dim, hidden):
        raise ValueError("w_folded must be [2, 3*heads*head_dim, hidden]")
    if frames is not None:
        _need(frames, "frames", torch.int32, 1)
    if out is None:
        out = tuple(torch.empty((T, heads, head_dim), dtype=torch.bfloat16, device=x.device) for _ in range(3))
    for name, t in zip("qkv", out):
        _need(t, name, torch.bfloat16, 3)
        if t.shape != (T, heads, head_dim):
            raise ValueError(f"{name} must be [T, heads, head_dim]")
    q, k, v = out
    fr = _ptr(frames) if frames is not None else None
    if events is None:
        _check(lib().mf_qkv_rmsnorm(_ptr(x), _ptr(w_folded), _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len), fr, n, T,
                                    hidden, heads, head_dim, float(eps), _ptr(q), _ptr(k), _ptr(v), _stream(stream)))
    else:
        arr = (ctypes.c_void_p * 3)(*events)
        _check(lib().mf_qkv_rmsnorm_profiled(_ptr(x), _ptr(w_folded), _ptr(cu_seqlens), _ptr(grid_hw),
                                             _ptr(text_len), fr, n, T, hidden, heads, head_dim, float(eps), _ptr(q),
                                             _ptr(k), _ptr(v), ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))
    return q, k, v


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() if t is not None and t.numel() > 0 else None for t in ts])


def _stream_args(text, image, joint, grid_hw, text_len, cu_seqlens, frames):
    n = len(joint)
    if not 1 <= n <= 4 or len(text) != n or len(image) != n:
        raise ValueError("1 to 4 tensors, the same number of text, image and joint tensors")
    ref = joint[0]
    _need(ref, "joint", ndim=3)
    if ref.dtype not in _DTYPES:
        raise ValueError("tensors must be bfloat16 or float32")
    T, H, D = ref.shape
    Tt = text[0].shape[0]
    for name, group, rows in (("joint", joint, T), ("text", text, Tt), ("image", image, T - Tt)):
        for t in group:
            _need(t, name, ref.dtype, 3)
            if t.shape != (rows, H, D):
                raise ValueError(f"{name} tensors must be [{rows}, {H}, {D}]")
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(grid_hw, "grid_hw", torch.int32, 2)
    _need(text_len, "text_len", torch.int32, 1)
    if frames is not None:
        _need(frames, "frames", torch.int32, 1)
    return grid_hw.shape[0], T, Tt, H, D, ref.dtype


def pack_joint(text, image, cu_seqlens, grid_hw, text_len, frames=None, out=None, stream=None):
    """Joint packed rows from the text and image streams (mf_pack_joint).

    text: tensors [sum T_i, H, d]; image: tensors [T - sum T_i, H, d] (one per
    tensor moved, up to 4, e.g. (q, k, v)). Returns the joint tensors [T, H, d]."""
    text, image = list(text), list(image)
    T = int(text[0].shape[0] + image[0].shape[0])
    if out is None:
        out = [torch.empty((T,) + tuple(text[0].shape[1:]), dtype=text[0].dtype, device=text[0].device)
               for _ in text]
    out = list(out)
    n, T, Tt, H, D, dt = _stream_args(text, image, out, grid_hw, text_len, cu_seqlens, frames)
    _check(lib().mf_pack_joint(len(out), _ptr_array(text), _ptr_array(image), _ptr_array(out), _ptr(cu_seqlens),
                               _ptr(grid_hw), _ptr(text_len), _ptr(frames) if frames is not None else None, n, T, Tt,
                               H, D, _DTYPES[dt], _stream(stream)))
    return out


def unpack_joint(joint, text_tokens: int, cu_seqlens, grid_hw, text_len, frames=None, out=None, stream=None):
    """Text and image streams from joint rows (mf_unpack_joint). Returns (text list, image list)."""
    joint = list(joint)
    T = int(joint[0].shape[0])
    if out is None:
        mk = lambda rows: [torch.empty((rows,) + tuple(j.shape[1:]), dtype=j.dtype, device=j.device)  # noqa: E731
                           for j in joint]
        out = (mk(text_tokens), mk(T - text_tokens))
    text, image = list(out[0]), list(out[1])
    n, T, Tt, H, D, dt = _stream_args(text, image, joint, grid_hw, text_len, cu_seqlens, frames)
    _check(lib().mf_unpack_joint(len(joint), _ptr_array(joint), _ptr_array(text), _ptr_array(image),
                                 _ptr(cu_seqlens), _ptr(grid_hw), _ptr(text_len),
                                 _ptr(frames) if frames is not None else None, n, T, Tt, H, D, _DTYPES[dt],
                                 _stream(stream)))
    return text, image


def get_device_error(stream=None) -> int:
    """Synchronizes and returns the device-side check status (MF_OK or MF_ERR_METADATA)."""
    return int(lib().mf_get_device_error(_stream(stream)))


def get_workspace_error(workspace, stream=None) -> int:
    return int(lib().mf_get_workspace_error(_ptr(workspace), _stream(stream)))


def last_error() -> str:
    return lib().mf_last_error().decode()
