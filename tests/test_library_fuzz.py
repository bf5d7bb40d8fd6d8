"""Seeded argument fuzz of every C-ABI entry point, host side only.

Each function in the binding's declaration table is called many times with
arguments drawn per parameter: mostly plausible values (disjoint aligned
fake device addresses, small batches, supported sizes), each replaced with
probability 0.15 by an edge value: null, misaligned or repeated (so
overlapping) addresses; sizes at and around the documented limits, zero,
negative and huge; special floats (0, negative, NaN, inf). The library must never crash and must return one of the documented
status codes with a message. Without a GPU every call that passes the host
checks stops at the device query (MF_ERR_HIP), so no fake address is ever
dereferenced; on a machine with a GPU such a call could reach a kernel, so the
test only runs where no device is present.
"""
import ctypes
import math
import random
import zlib

import pytest
import torch

from text_image_diffusion_varlen_amd import binding

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="random device addresses need a host without a GPU")

ERRORS = {binding.MF_ERR_INVALID_ARG, binding.MF_ERR_METADATA, binding.MF_ERR_UNSUPPORTED, binding.MF_ERR_HIP,
          binding.MF_ERR_OOM}
I32 = [0, 1, 2, 3, 7, 16, 24, 48, 64, 96, 128, 256, 4096, 4097, 65536, 2**31 - 1, -1, -2**31]
I64 = [0, 1, 64, 288, 4352, 2**31 - 1, 2**31, 2**40, -1, -2**40]
F32 = [0.0, 1e-6, 0.5, 5.0, 10000.0, -1.0, math.nan, math.inf, -math.inf]
SZ = [0, 1, 1 << 20, 1 << 40]


# Plausible values: what a correct call passes (disjoint aligned buffers,
# small batches, supported head sizes), so that some calls pass every check.
PLAUSIBLE = {ctypes.c_int32: [0, 1, 2, 32, 64, 128, 256], ctypes.c_int64: [288, 4352],
             ctypes.c_float: [5.0, 0.25, 1e-6, 10000.0], ctypes.c_size_t: [1 << 40]}


def _pointer(rng):
    k = rng.randint(1, 12)
    return rng.choice([None, 0x100000 * k, 0x100000 * k, 0x100000 * k + 4, 0x100000 * k + 8])


def _draw(rng, t, position):
    if rng.random() < 0.85:  # plausible
        if t is ctypes.c_void_p:
            return 0x40000000 * (position + 1)  # 1 GiB apart: never overlapping
        return rng.choice(PLAUSIBLE[t])
    if t is ctypes.c_void_p:
        return _pointer(rng)
    if t is ctypes.c_int32:
        return rng.choice(I32)
    if t is ctypes.c_int64:
        return rng.choice(I64)
    if t is ctypes.c_float:
        return rng.choice(F32)
    if t is ctypes.c_size_t:
        return rng.choice(SZ)
    raise AssertionError(f"no generator for {t}")


# Arguments that are host arrays of device pointers (position in the argument list).
HOST_ARRAYS = {"mf_pack_joint": {1, 2, 3}, "mf_unpack_joint": {1, 2, 3}}
# Arguments that are host pointers to mf_tensor descriptors.
DESCRIPTORS = {"mf_attn_packed_strided": {0, 1, 2, 7}}
STRIDES = [0, 1, 8, 64, 128, 3072, 9216, 2**31, -8, 2**40]


def _descriptor(rng, position):
    """A host mf_tensor: plausible fields (a contiguous bf16 4352 x 24 x 128
    tensor at a disjoint fake address), each replaced with probability 0.15 by
    an edge value; or a null descriptor."""
    if rng.random() < 0.1:
        return None
    pick = lambda plausible, edge: plausible if rng.random() < 0.85 else rng.choice(edge)  # noqa: E731
    d = binding.MfTensor(pick(0x40000000 * (position + 1), [None, 0x100004, 0x100000]),
                         pick(0, I32), pick(4352, I32), pick(24, I32), pick(128, I32),
                         pick(24 * 128, STRIDES), pick(128, STRIDES))
    return ctypes.pointer(d)


def _host_array(rng, position):
    """A host array of 4 device pointers: plausible (disjoint, aligned) entries,
    each replaced with probability 0.15 by an edge address; or a null array."""
    if rng.random() < 0.1:
        return None
    entries = [0x40000000 * (8 * position + i + 1) if rng.random() < 0.85 else _pointer(rng) for i in range(4)]
    return (ctypes.c_void_p * 4)(*entries)


def _functions():
    lib = binding.lib()
    return [(name, getattr(lib, name)) for name in binding.header_functions()]


@pytest.mark.parametrize("name", sorted(binding.header_functions()))
def test_entry_point_returns_documented_codes(name):
    fn = dict(_functions())[name]
    rng = random.Random(zlib.crc32(name.encode()))
    for _ in range(600):
        args = [_host_array(rng, i) if i in HOST_ARRAYS.get(name, ()) else
                _descriptor(rng, i) if i in DESCRIPTORS.get(name, ()) else _draw(rng, t, i)
                for i, t in enumerate(fn.argtypes)]
        r = fn(*args)
        if fn.restype is ctypes.c_size_t:
            assert 0 <= r < (1 << 50), (name, args, r)
        elif fn.restype is ctypes.c_char_p:
            assert isinstance(r, bytes)
        elif name == "mf_version":
            assert r == 100
        else:
            assert r in ERRORS, (name, args, r)
            assert binding.last_error() != "", (name, args)
