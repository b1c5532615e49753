"""Seeded, counter-based synthetic inputs shared by the oracle side and the GPU side.

The generator definition lives in ``synth_core.h``.  This module holds no part of
the decoder arithmetic: it only turns (seed, tensor name, element index) into
bf16 values or int32 token ids, on the host (numpy) or directly into device
memory (for large tensors).  bf16 tensors are carried as ``numpy.uint16``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_host = None
_dev = None


def _lib_host():
    global _host
    if _host is None:
        if not os.path.exists(_build.HOST_SO):
            _build.build_host()
        lib = ctypes.CDLL(_build.HOST_SO)
        lib.synth_stream_id.restype = ctypes.c_uint64
        lib.synth_stream_id.argtypes = [ctypes.c_char_p]
        i64, u64 = ctypes.c_int64, ctypes.c_uint64
        lib.synth_normal_bf16_3d.argtypes = [u64, u64, u64, i64, i64, i64, ctypes.c_float,
                                             ctypes.c_float, ctypes.c_void_p, i64, i64, i64,
                                             ctypes.c_int]
        lib.synth_uniform_i32_3d.argtypes = [u64, u64, u64, i64, i64, i64, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, i64, i64, i64,
                                             ctypes.c_int]
        _host = lib
    return _host


def _lib_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(_build.DEVICE_SO):
            _build.build_device()
        lib = ctypes.CDLL(_build.DEVICE_SO)
        i64, u64 = ctypes.c_int64, ctypes.c_uint64
        lib.synth_normal_bf16_3d_device.argtypes = [u64, u64, u64, i64, i64, i64, ctypes.c_float,
                                                    ctypes.c_float, ctypes.c_void_p, i64, i64,
                                                    i64, ctypes.c_void_p]
        lib.synth_normal_bf16_3d_device.restype = ctypes.c_int
        lib.synth_uniform_i32_3d_device.argtypes = [u64, u64, u64, i64, i64, i64, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_void_p, i64, i64,
                                                    i64, ctypes.c_void_p]
        lib.synth_uniform_i32_3d_device.restype = ctypes.c_int
        _dev = lib
    return _dev


def nthreads():
    n = os.environ.get("SYNTH_THREADS")
    if n:
        return max(1, int(n))
    return max(1, min(16, os.cpu_count() or 1))


def stream_id(name: str) -> int:
    return _lib_host().synth_stream_id(name.encode())


def _as3(shape):
    shape = tuple(int(s) for s in shape)
    if len(shape) == 0:
        return 1, 1, 1
    cols = shape[-1]
    rows = shape[-2] if len(shape) >= 2 else 1
    batch = int(np.prod(shape[:-2])) if len(shape) >= 3 else 1
    return batch, rows, cols


def normal_bf16(seed, name, shape, mean=0.0, std=1.0, offset=0):
    """Host bf16 (as uint16) tensor of the given logical shape."""
    out = np.empty(shape, dtype=np.uint16)
    b, r, c = _as3(shape)
    _lib_host().synth_normal_bf16_3d(seed, stream_id(name), offset, b, r, c, mean, std,
                                     out.ctypes.data, r * c, c, 1, nthreads())
    return out


def uniform_i32(seed, name, shape, lo, hi, offset=0):
    out = np.empty(shape, dtype=np.int32)
    b, r, c = _as3(shape)
    _lib_host().synth_uniform_i32_3d(seed, stream_id(name), offset, b, r, c, lo, hi,
                                     out.ctypes.data, r * c, c, 1, nthreads())
    return out


def normal_bf16_strided_host(seed, name, out, logical, strides, mean=0.0, std=1.0, offset=0):
    """Write logical [batch, rows, cols] values into ``out`` (uint16 array) at element
    strides ``(ld_b, ld_r, ld_c)``."""
    b, r, c = logical
    _lib_host().synth_normal_bf16_3d(seed, stream_id(name), offset, b, r, c, mean, std,
                                     out.ctypes.data, strides[0], strides[1], strides[2],
                                     nthreads())
    return out


def normal_bf16_device(tensor, seed, name, mean=0.0, std=1.0, offset=0, logical=None,
                       strides=None, stream=None):
    """Fill a device tensor (dtype bfloat16) in place on ``stream`` (default: torch's
    current stream).  ``logical`` / ``strides`` as in the host strided variant; by
    default the tensor is filled contiguously in its own logical order."""
    import torch
    if logical is None:
        logical = _as3(tensor.shape)
        strides = (logical[1] * logical[2], logical[2], 1)
    if stream is None:
        stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _lib_dev().synth_normal_bf16_3d_device(seed, stream_id(name), offset, logical[0],
                                                logical[1], logical[2], mean, std,
                                                tensor.data_ptr(), strides[0], strides[1],
                                                strides[2], stream)
    if rc != 0:
        raise RuntimeError("synth device generator launch failed")
    return tensor


def uniform_i32_device(tensor, seed, name, lo, hi, offset=0, stream=None):
    import torch
    b, r, c = _as3(tensor.shape)
    if stream is None:
        stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _lib_dev().synth_uniform_i32_3d_device(seed, stream_id(name), offset, b, r, c, lo, hi,
                                                tensor.data_ptr(), r * c, c, 1, stream)
    if rc != 0:
        raise RuntimeError("synth device generator launch failed")
    return tensor


def bf16_to_f32(u16):
    """Exact widening of bf16 bits (uint16 array) to float32."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x):
    """Round-to-nearest-even narrowing of float32 to bf16 bits (uint16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)
