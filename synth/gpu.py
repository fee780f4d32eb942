"""Device-side fills of synthetic blob pools (same bytes as synth.fill_blob)."""

from __future__ import annotations

import ctypes
import os

from . import Geometry, SHARED_BLOB_ID

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(HERE, "libmoe_synth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        L.synth_fill_blobs.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        L.synth_fill_blobs.restype = ctypes.c_int
        _lib = L
    return _lib


def fill_blobs(geo: Geometry, dst_ptr: int, n_blobs: int, seed: int, layer: int, blob_id0: int = 0,
               shared: bool = False, stream: int = 0) -> None:
    """Fill n_blobs consecutive slots starting at device address dst_ptr."""
    inter = geo.shared_inter if shared else geo.inter
    stride = geo.shared_stride if shared else geo.blob_stride
    bid = SHARED_BLOB_ID if shared else blob_id0
    rc = lib().synth_fill_blobs(dst_ptr, stride, n_blobs, geo.hidden, inter, geo.bits,
                                1 if geo.sb == "f32" else 0, seed, layer, bid, stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_blobs failed with {rc}")
