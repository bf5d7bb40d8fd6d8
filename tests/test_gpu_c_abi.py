"""The library used from plain C, with no Python or torch in the process.

A C99 program (built here with gcc against mf_attn.h and the HIP runtime)
reads a seeded packed batch from files, allocates device buffers with
hipMalloc, builds cu_seqlens with mf_build_metadata, runs mf_attn_packed on
the null stream, checks mf_get_device_error and writes the output back. The
output must meet the bf16 parity bars against the fp64 oracle.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import attention
from text_image_diffusion_varlen_amd import binding, workloads

from gpu_common import check_close

pytestmark = pytest.mark.gpu

C_SOURCE = r"""
#include <stdio.h>
#include <stdlib.h>
#include "mf_attn.h"

static void* slurp(const char* path, size_t bytes) {
  void* p = malloc(bytes);
  FILE* f = fopen(path, "rb");
  if (!p || !f || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "read %s\n", path); exit(2); }
  fclose(f);
  return p;
}

static void* upload(const void* h, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "upload\n");
    exit(3);
  }
  return d;
}

int main(int argc, char** argv) {
  if (argc != 6) return 1;
  const int n = atoi(argv[2]), heads = atoi(argv[4]), d = atoi(argv[5]);
  const long long T = atoll(argv[3]);
  char path[4096];
  const size_t tb = (size_t)T * heads * d * 2;
  snprintf(path, sizeof path, "%s/q.bin", argv[1]); void* q = upload(slurp(path, tb), tb);
  snprintf(path, sizeof path, "%s/k.bin", argv[1]); void* k = upload(slurp(path, tb), tb);
  snprintf(path, sizeof path, "%s/v.bin", argv[1]); void* v = upload(slurp(path, tb), tb);
  snprintf(path, sizeof path, "%s/grid.bin", argv[1]); int32_t* grid = upload(slurp(path, 8 * (size_t)n), 8 * (size_t)n);
  snprintf(path, sizeof path, "%s/text.bin", argv[1]); int32_t* text = upload(slurp(path, 4 * (size_t)n), 4 * (size_t)n);
  int32_t *cu = NULL, *pos = NULL, *seg = NULL;
  void* out = NULL;
  if (hipMalloc((void**)&cu, 4 * ((size_t)n + 1)) != hipSuccess || hipMalloc((void**)&pos, 8 * (size_t)T) != hipSuccess ||
      hipMalloc((void**)&seg, 4 * (size_t)T) != hipSuccess || hipMalloc(&out, tb) != hipSuccess) return 4;
  int rc = mf_build_metadata(n, grid, text, cu, pos, seg, T, NULL);
  if (rc == MF_OK) rc = mf_attn_packed(q, k, v, cu, grid, text, out, n, T, heads, d, MF_BF16, NULL);
  if (rc == MF_OK) rc = mf_get_device_error(NULL);
  if (rc != MF_OK) { fprintf(stderr, "mfattn %d: %s\n", rc, mf_last_error()); return 5; }
  void* h = malloc(tb);
  if (!h || hipMemcpy(h, out, tb, hipMemcpyDeviceToHost) != hipSuccess) return 6;
  snprintf(path, sizeof path, "%s/out.bin", argv[1]);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(h, 1, tb, f) != tb) return 7;
  fclose(f);
  return 0;
}
"""


def test_attention_from_a_c_program():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    w = workloads.make_custom([[12, 20], [1, 40], [9, 9]], [33, 0, 100], heads=2, head_dim=128, dtype="bf16",
                              seed=40, name="c_abi")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out_dir = os.path.join(root, "_build", "c_abi_gpu")  # build folder, kept out of the repository
    os.makedirs(out_dir, exist_ok=True)
    for name, a in (("q", w.q), ("k", w.k), ("v", w.v)):
        workloads.f32_to_bf16_bits(a).tofile(os.path.join(out_dir, f"{name}.bin"))
    w.grid_hw.astype(np.int32).tofile(os.path.join(out_dir, "grid.bin"))
    w.text_len.astype(np.int32).tofile(os.path.join(out_dir, "text.bin"))
    src, exe = os.path.join(out_dir, "main.c"), os.path.join(out_dir, "main")
    with open(src, "w") as f:
        f.write(C_SOURCE)
    lib_dir = os.path.dirname(binding.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                        "-I", "/opt/rocm/include", src, "-L", lib_dir, "-lmfattn", "-L", "/opt/rocm/lib", "-lamdhip64",
                        f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    print(f"c abi: T={w.tokens} n={w.n_seg}", flush=True)
    run = subprocess.run([exe, out_dir, str(w.n_seg), str(w.tokens), str(w.heads), str(w.head_dim)],
                         capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    bits = np.fromfile(os.path.join(out_dir, "out.bin"), dtype=np.uint16).reshape(w.q.shape)
    got = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    check_close(got, attention.joint_attention(w.q, w.k, w.v, w.grid_hw, w.text_len), "bf16")
