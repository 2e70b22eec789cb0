"""ctypes binding of libsplitkv_probe.so (include/read_probe.h): a plain
streaming read of device memory that the benchmark times beside the decode.
Measurement only; the decode path never calls it."""

from __future__ import annotations

import ctypes
import os

from ._lib import one_hip_runtime

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(HERE, "libsplitkv_probe.so")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        one_hip_runtime()
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is missing: build it with "
                               "`python -m split_kv_paged_page_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(PROBE_PATH)
        L.splitkv_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p]
        L.splitkv_read_probe.restype = ctypes.c_int32
        _lib = L
    return _lib


def read_probe(buf: int, nbytes: int, workgroups: int, sink: int, stream: int = 0) -> None:
    """Enqueue one read of `nbytes` device bytes at address `buf` on `stream`;
    `sink` is a device buffer of at least `workgroups` 32-bit words."""
    rc = lib().splitkv_read_probe(buf, nbytes, workgroups, sink, stream)
    if rc != 0:
        raise RuntimeError(f"splitkv_read_probe failed with status {rc}")
