"""Packed joint text+image attention with 2D RoPE for MI355X (gfx950).

The compute path lives in the HIP library ``libmfattn.so`` (sources in
``csrc/``); ``binding`` is its thin ctypes wrapper. ``workloads`` draws seeded
synthetic inputs.
"""
__version__ = "0.1.0"
