"""Mamba-3 selective SSM scan for MI355X (gfx950).

The compute lives in ``libm3scan.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/m3scan.h``).  ``state_space_sequence_scan_amd.m3scan``
is the thin Python binding (argument marshalling only; PyTorch supplies device
memory and the current HIP stream).  Importing this package does not load the
library; the first call does, and raises if it is missing.
"""
from .configs import CONFIGS, ScanConfig  # noqa: F401

__all__ = ["CONFIGS", "ScanConfig"]


def __getattr__(name):
    if name in ("prefill", "decode_step", "DecodeState", "lib", "workspace_size"):
        from . import m3scan
        return getattr(m3scan, name)
    raise AttributeError(name)
