"""Failure detection and debugging aids of the library, each in a child
process so that the environment switch is read fresh and no workspace of an
earlier test is already large enough:

- MF_FAULT_OOM=1 makes the next workspace allocation fail: the call returns
  MF_ERR_OOM with a message and launches nothing; once unset, the same call
  succeeds and meets the parity bars.
- MF_DEBUG=1 synchronizes after every stage and checks the launch, device
  faults and the device flags, so a metadata mismatch is reported by the call
  itself (MF_ERR_METADATA, naming the stage) instead of only by
  mf_get_device_error; consistent calls still succeed with the same bits as
  without it.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_PRELUDE = r'''
import os, sys
sys.path.insert(0, {root!r})
sys.path.insert(0, os.path.join({root!r}, "tests"))
import numpy as np, torch
from oracle import attention
from text_image_diffusion_varlen_amd import binding, workloads
from gpu_common import check_close, device_inputs, to_f64
torch.cuda.set_device(0)
w = workloads.make_custom([[6, 11], [3, 3], [1, 40]], [20, 0, 5], heads=4, head_dim=128, dtype="bf16", seed=11)
q, k, v, grid, text = device_inputs(w)
cu, _, _ = binding.build_metadata(grid, text, w.tokens)
torch.cuda.synchronize()
ref = attention.joint_attention(w.q, w.k, w.v, w.grid_hw, w.text_len)
'''


def _child(body, **env):
    code = _PRELUDE.format(root=ROOT) + body
    r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, **env), capture_output=True, text=True,
                       timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-2000:]
    assert "CHILD_OK" in r.stdout


def test_injected_allocation_failure():
    _child(r'''
try:
    binding.attn_packed(q, k, v, cu, grid, text)
    raise SystemExit("expected MF_ERR_OOM")
except binding.MFError as e:
    assert e.code == binding.MF_ERR_OOM, e
    assert "injected" in str(e), e
    print("oom:", e)
os.environ.pop("MF_FAULT_OOM")
out = binding.attn_packed(q, k, v, cu, grid, text)
torch.cuda.synchronize()
assert binding.get_device_error() == binding.MF_OK, binding.last_error()
check_close(to_f64(out), ref, "bf16")
print("CHILD_OK")
''', MF_FAULT_OOM="1")


def test_debug_mode_reports_errors_at_the_call():
    _child(r'''
out = binding.attn_packed(q, k, v, cu, grid, text)
torch.cuda.synchronize()
check_close(to_f64(out), ref, "bf16")
bad_cu = torch.tensor([0, 17, 26, w.tokens], dtype=torch.int32, device="cuda")
sentinel = torch.full_like(q, 7.0)
try:
    binding.attn_packed(q, k, v, bad_cu, grid, text, out=sentinel)
    raise SystemExit("expected MF_ERR_METADATA from the call")
except binding.MFError as e:
    assert e.code == binding.MF_ERR_METADATA, e
    assert "metadata" in str(e) or "meta_kernel" in str(e), e
    print("metadata:", e)
torch.cuda.synchronize()
assert torch.all(sentinel == 7.0), "a failed metadata check wrote output"
bad_grid = torch.tensor([[6, 11], [3, 3], [1, 600]], dtype=torch.int32, device="cuda")
try:
    binding.build_metadata(bad_grid, text, w.tokens)
    raise SystemExit("expected MF_ERR_METADATA from mf_build_metadata")
except binding.MFError as e:
    assert e.code == binding.MF_ERR_METADATA, e
    print("build_metadata:", e)
out2 = binding.attn_packed(q, k, v, cu, grid, text)
torch.cuda.synchronize()
assert torch.equal(out, out2)
assert binding.get_device_error() == binding.MF_OK, binding.last_error()
print("CHILD_OK")
''', MF_DEBUG="1")
