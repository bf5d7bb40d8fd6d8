"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports every
function the header declares, and rejects bad arguments before touching a device."""
import ctypes
import subprocess

import pytest

from text_image_diffusion_varlen_amd import binding


def test_library_loads_and_exports_header_symbols():
    lib = binding.lib()
    names = binding.header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= exported
    assert binding.version() == 100


def test_mfma_probe_library_loads_and_rejects_bad_arguments():
    """The benchmark's MFMA-rate aid is a separate library; its entry point
    checks its arguments on the host (hipErrorInvalidValue = 1)."""
    import os

    path = os.path.join(os.path.dirname(binding.LIB_PATH), "libmfprobe.so")
    lib = ctypes.CDLL(path)
    f = lib.mf_probe_mfma_loop
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert f(None, 0, 1, 1, None) == 1
    buf = ctypes.create_string_buffer(16)
    assert f(ctypes.cast(buf, ctypes.c_void_p), 2, 1, 1, None) == 1
    assert f(ctypes.cast(buf, ctypes.c_void_p), 0, 0, 1, None) == 1
    assert f(ctypes.cast(buf, ctypes.c_void_p), 1, 1, 0, None) == 1


def test_workspace_bytes():
    import torch
    wb = binding.workspace_bytes
    tensor = 4352 * 24 * 128
    # bf16: K~ and V~^T (queries are rotated in the kernel) and 512 partial-result
    # slots of 256 rows x (128 + 2) floats; fp32: Q~, K~ and V, no partials
    partials = 512 * 256 * 130 * 4
    assert 2 * tensor * 2 + partials < wb(4352, 24, 128, torch.bfloat16, 1) < 3 * tensor * 2 + partials
    assert 3 * tensor * 4 < wb(4352, 24, 128, torch.float32, 1) < 4 * tensor * 4
    lib = binding.lib()
    assert lib.mf_workspace_bytes(100, 2, 96, 0, 1) == 0  # unsupported head_dim
    assert lib.mf_workspace_bytes(100, 2, 64, 7, 1) == 0  # unknown dtype
    assert lib.mf_workspace_bytes(0, 2, 64, 0, 1) == 0
    assert lib.mf_workspace_bytes(100, 2, 64, 0, 5000) == 0
    # backward: seven bf16 operand buffers, the row statistics, 512 slots of
    # 128 keys x d fp32 partial dV and dK and 512 slots of 256 rows x d fp32
    # partial dQ for the split last rounds
    for d in (64, 128):
        t = 4352 * 24 * d * 2
        slots = 512 * 2 * 128 * d * 4 + 512 * 256 * d * 4
        assert 7 * t + slots < lib.mf_bwd_workspace_bytes(4352, 24, d, 1) < 8 * t + slots
    assert lib.mf_bwd_workspace_bytes(4352, 24, 96, 1) == 0
    assert lib.mf_bwd_workspace_bytes(0, 24, 128, 1) == 0


def _call(q=0x10000, k=0x20000, v=0x30000, cu=0x40000, grid=0x50000, text=0x60000, out=0x70000,
          n=1, T=64, H=2, D=64, dtype=0):
    lib = binding.lib()
    P = ctypes.c_void_p
    return lib.mf_attn_packed(P(q), P(k), P(v), P(cu), P(grid), P(text), P(out), n, T, H, D, dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(q=0), binding.MF_ERR_INVALID_ARG),
    (dict(out=0), binding.MF_ERR_INVALID_ARG),
    (dict(n=0), binding.MF_ERR_INVALID_ARG),
    (dict(n=5000), binding.MF_ERR_INVALID_ARG),
    (dict(T=0), binding.MF_ERR_INVALID_ARG),
    (dict(T=2**31), binding.MF_ERR_INVALID_ARG),
    (dict(H=0), binding.MF_ERR_INVALID_ARG),
    (dict(D=96), binding.MF_ERR_UNSUPPORTED),
    (dict(dtype=3), binding.MF_ERR_UNSUPPORTED),
    (dict(out=0x10000 + 64), binding.MF_ERR_INVALID_ARG),  # out overlaps q
    (dict(out=0x40000), binding.MF_ERR_INVALID_ARG),  # out overlaps the offsets
    (dict(q=0x10004), binding.MF_ERR_INVALID_ARG),  # misaligned
])
def test_attn_rejects_bad_arguments_on_host(kwargs, code):
    assert _call(**kwargs) == code
    assert binding.last_error() != ""


def test_other_entry_points_reject_bad_arguments():
    lib = binding.lib()
    P = ctypes.c_void_p
    assert lib.mf_build_metadata(0, P(1), P(2), P(3), P(4), P(5), 10, None) == binding.MF_ERR_INVALID_ARG
    assert lib.mf_build_metadata(1, None, P(2), P(3), P(4), P(5), 10, None) == binding.MF_ERR_INVALID_ARG
    assert lib.mf_rope_2d(P(16), P(4096), P(64), 10, 1, 96, 0, 10000.0, None) == binding.MF_ERR_UNSUPPORTED
    assert lib.mf_rope_2d(P(16), P(4096), P(64), 10, 1, 64, 0, 0.5, None) == binding.MF_ERR_INVALID_ARG
    assert lib.mf_rope_2d(P(16), P(32), P(64), 10, 1, 64, 0, 10000.0, None) == binding.MF_ERR_INVALID_ARG
    ws = lib.mf_workspace_bytes(64, 2, 64, 0, 1)
    assert lib.mf_attn_packed_ws(P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x50000), P(0x60000),
                                 P(0x70000), 1, 64, 2, 64, 0, None, ws, None) == binding.MF_ERR_INVALID_ARG
    assert lib.mf_attn_packed_ws(P(0x10000), P(0x20000), P(0x30000), P(0x40000), P(0x50000), P(0x60000),
                                 P(0x70000), 1, 64, 2, 64, 0, P(0x1000000), ws - 1, None) == binding.MF_ERR_INVALID_ARG
    assert lib.mf_get_workspace_error(None, None) == binding.MF_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros((4, 1, 64))
    with pytest.raises(ValueError):
        binding.rope_2d(x, torch.zeros((4, 2), dtype=torch.int32))


def test_cfg_step_rejects_bad_arguments_on_host():
    lib = binding.lib()
    P = ctypes.c_void_p

    def call(z=0x10000, v=0x200000, n_seg=2, T=40, n_img=1, img=16, C=8, dtype=0, s=5.0, dt=0.25, cs=0x300000):
        return lib.mf_rf_cfg_euler_step(P(z), P(v), P(0x400000), P(0x500000), P(0x600000), n_seg, T, P(cs),
                                        P(0x700000), n_img, img, C, dtype, s, dt, None)

    bad = binding.MF_ERR_INVALID_ARG
    assert call(z=0) == bad
    assert call(cs=0) == bad
    assert call(n_seg=0) == bad
    assert call(n_img=0) == bad
    assert call(n_img=5000) == bad
    assert call(T=0) == bad
    assert call(img=0) == bad
    assert call(C=12) == binding.MF_ERR_UNSUPPORTED
    assert call(C=0) == binding.MF_ERR_UNSUPPORTED
    assert call(dtype=5) == binding.MF_ERR_UNSUPPORTED
    assert call(s=float("nan")) == bad
    assert call(dt=float("inf")) == bad
    assert call(z=0x10004) == bad  # misaligned
    assert call(v=0x10000 + 64) == bad  # z overlaps v
    assert binding.last_error() != ""


def test_backward_3d_and_projection_reject_bad_arguments_on_host():
    lib = binding.lib()
    P = ctypes.c_void_p
    bad, uns = binding.MF_ERR_INVALID_ARG, binding.MF_ERR_UNSUPPORTED
    a = [P(0x10000 * (i + 1)) for i in range(12)]
    # backward: fp32 is unsupported, null d_out rejected
    assert lib.mf_attn_packed_bwd(*a, 1, 64, 2, 64, 1, None) == uns
    args = list(a)
    args[4] = None
    assert lib.mf_attn_packed_bwd(*args, 1, 64, 2, 64, 0, None) == bad
    # 3D forward: split must be even, non-negative and sum to head_dim; frames required
    f3 = [P(0x100000 * (i + 1)) for i in range(7)]
    assert lib.mf_attn_packed_3d(*f3, 30, 30, 2, P(0x900000), None, 1, 64, 2, 64, 0, None) == bad
    assert lib.mf_attn_packed_3d(*f3, 31, 31, 2, P(0x900000), None, 1, 64, 2, 64, 0, None) == bad
    f3[6] = None
    assert lib.mf_attn_packed_3d(*f3, 24, 24, 16, P(0x900000), None, 1, 64, 2, 64, 0, None) == bad
    assert lib.mf_build_metadata_3d(1, P(1), P(2), None, P(3), P(4), P(5), 10, None) == bad
    assert lib.mf_rope_3d(P(16), P(4096), P(64), 10, 1, 64, 0, 10000.0, 24, 24, 18, None) == bad
    # projection: hidden must be a multiple of 64, heads * head_dim a multiple of 256
    q = [P(0x1000000 * (i + 1)) for i in range(6)]
    o = [P(0x9000000 + 0x1000000 * i) for i in range(3)]
    assert lib.mf_qkv_rmsnorm(*q, 1, 10, 96, 2, 128, 1e-6, *o, None) == uns
    assert lib.mf_qkv_rmsnorm(*q, 1, 10, 128, 3, 64, 1e-6, *o, None) == uns
    assert lib.mf_qkv_rmsnorm(*q, 1, 10, 128, 2, 128, -1.0, *o, None) == bad
    assert lib.mf_qkv_fold_weights(P(16), P(32), P(48), P(64), 96, 2, 128, P(4096), None) == uns
    assert binding.last_error() != ""


def test_header_is_c99_and_the_library_links_from_c():
    """The boundary is a C ABI: a C99 program that includes only mf_attn.h (and
    the HIP runtime API header it names) compiles without warnings, links
    against the built library and runs its host-side calls without a GPU."""
    import os
    import shutil

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = os.path.join(root, "_build", "c_abi")  # build folder, kept out of the repository
    os.makedirs(out, exist_ok=True)
    src = os.path.join(out, "main.c")
    with open(src, "w") as f:
        f.write(
            "#include <stdio.h>\n"
            "#include \"mf_attn.h\"\n"
            "int main(void) {\n"
            "  size_t ws = mf_workspace_bytes(4352, 24, 128, MF_BF16, 1);\n"
            "  int bad = mf_attn_packed(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 64, 2, 64, MF_BF16, NULL);\n"
            "  printf(\"%d %zu %d %d\\n\", mf_version(), ws, bad, mf_last_error()[0] != 0);\n"
            "  return 0;\n"
            "}\n")
    lib_dir = os.path.dirname(binding.LIB_PATH)
    exe = os.path.join(out, "main")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include", src, "-L", lib_dir,
                        "-lmfattn", f"-Wl,-rpath,{lib_dir}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    version, ws, bad, has_msg = run.stdout.split()
    assert int(version) == 100 and int(ws) == binding.lib().mf_workspace_bytes(4352, 24, 128, 0, 1)
    assert int(bad) == binding.MF_ERR_INVALID_ARG and has_msg == "1"
