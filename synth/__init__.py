"""Seeded synthetic inputs for the gradient-bucket reduction workloads.

Input tooling only. Nothing in here computes any part of the reduction; the
CPU oracle and the GPU path both draw their inputs from it. The host
generator (``synth_host.c``) and the device generator (``synth_dev.hip``)
implement one counter-based definition (SplitMix64 at a counter, see the
header of ``synth_host.c``) and agree bit for bit.

Workload shapes live in :mod:`synth.workloads`.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

_u64, _u32, _i32, _f32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_float
_vp = ctypes.c_void_p

_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_normal_bf16.argtypes = [_u64, _u64, _u64, _u64, _f32, _u32, _f32, _vp]
        lib.synth_points_normal_bf16.argtypes = [_u64, _vp, _vp, _u64, _f32, _u32, _f32, _vp]
        lib.synth_uniform_int_f32.argtypes = [_u64, _u64, _u64, _u64, _i32, _i32, _vp]
        lib.synth_uniform_int_bf16.argtypes = [_u64, _u64, _u64, _u64, _i32, _i32, _vp]
        lib.synth_words.argtypes = [_u64, _u64, _u64, _u64, _vp]
        for f in ("synth_normal_bf16", "synth_points_normal_bf16", "synth_uniform_int_f32",
                  "synth_uniform_int_bf16", "synth_words"):
            getattr(lib, f).restype = None
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_dev_normal_bf16.argtypes = [_u64, _u64, _u64, _u64, _f32, _u32, _f32, _vp, _vp]
        lib.synth_dev_uniform_int_f32.argtypes = [_u64, _u64, _u64, _u64, _i32, _i32, _vp, _vp]
        lib.synth_dev_uniform_int_bf16.argtypes = [_u64, _u64, _u64, _u64, _i32, _i32, _vp, _vp]
        for f in ("synth_dev_normal_bf16", "synth_dev_uniform_int_f32",
                  "synth_dev_uniform_int_bf16"):
            getattr(lib, f).restype = ctypes.c_int
        _dev = lib
    return _dev


def outlier_threshold(p: float) -> int:
    """Integer threshold t with P(hi32(word) < t) = t / 2^32 closest to p."""
    if p <= 0.0:
        return 0
    return min(int(math.floor(p * 2.0 ** 32)), 2 ** 32 - 1)


# ---------------------------------------------------------------- host side
def host_normal_bf16(seed, stream, start, count, sigma, outlier_p=0.0, outlier_mag=0.0):
    """bf16 bit patterns (uint16) of elements start..start+count-1 of a stream."""
    out = np.empty(int(count), dtype=np.uint16)
    if count:
        _load_host().synth_normal_bf16(seed, stream, start, count, sigma,
                                       outlier_threshold(outlier_p), outlier_mag,
                                       out.ctypes.data)
    return out


def host_points_normal_bf16(seed, streams, idx, sigma, outlier_p=0.0, outlier_mag=0.0):
    """bf16 bit patterns at arbitrary (stream, index) points."""
    streams = np.ascontiguousarray(streams, dtype=np.uint64)
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    assert streams.shape == idx.shape
    out = np.empty(idx.shape, dtype=np.uint16)
    if idx.size:
        _load_host().synth_points_normal_bf16(seed, streams.ctypes.data, idx.ctypes.data,
                                              idx.size, sigma, outlier_threshold(outlier_p),
                                              outlier_mag, out.ctypes.data)
    return out


def host_uniform_int_f32(seed, stream, start, count, lo, hi):
    out = np.empty(int(count), dtype=np.float32)
    if count:
        _load_host().synth_uniform_int_f32(seed, stream, start, count, lo, hi, out.ctypes.data)
    return out


def host_uniform_int_bf16(seed, stream, start, count, lo, hi):
    out = np.empty(int(count), dtype=np.uint16)
    if count:
        _load_host().synth_uniform_int_bf16(seed, stream, start, count, lo, hi, out.ctypes.data)
    return out


def host_words(seed, stream, start, count):
    out = np.empty(int(count), dtype=np.uint64)
    if count:
        _load_host().synth_words(seed, stream, start, count, out.ctypes.data)
    return out


def log_uniform_sizes(seed, n, hi=65536, stream=0xF4A6):
    """n sizes log-uniform in [1, hi]: floor(exp(u * ln(hi + 1))) clamped to [1, hi],
    with u = the top 53 bits of one generator word (host metadata, fp64)."""
    w = host_words(seed, stream, 0, n)
    out = []
    for x in w.tolist():
        u = (x >> 11) * 2.0 ** -53
        v = int(math.floor(math.exp(u * math.log(hi + 1))))
        out.append(min(max(v, 1), hi))
    return out


# -------------------------------------------------------------- device side
def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check_dev_tensor(t, itemsize):
    if not t.is_cuda or not t.is_contiguous() or t.element_size() != itemsize:
        raise ValueError("expected a contiguous CUDA tensor with %d-byte elements" % itemsize)


def dev_normal_bf16(t, seed, stream_id, start, sigma, outlier_p=0.0, outlier_mag=0.0,
                    stream=None):
    """Fill a contiguous 2-byte CUDA tensor with the generator's bf16 normals."""
    _check_dev_tensor(t, 2)
    rc = _load_dev().synth_dev_normal_bf16(seed, stream_id, start, t.numel(), sigma,
                                           outlier_threshold(outlier_p), outlier_mag,
                                           t.data_ptr(), _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_normal_bf16 failed ({rc})")


def dev_uniform_int_f32(t, seed, stream_id, start, lo, hi, stream=None):
    _check_dev_tensor(t, 4)
    rc = _load_dev().synth_dev_uniform_int_f32(seed, stream_id, start, t.numel(), lo, hi,
                                               t.data_ptr(), _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_uniform_int_f32 failed ({rc})")


def dev_uniform_int_bf16(t, seed, stream_id, start, lo, hi, stream=None):
    _check_dev_tensor(t, 2)
    rc = _load_dev().synth_dev_uniform_int_bf16(seed, stream_id, start, t.numel(), lo, hi,
                                                t.data_ptr(), _stream_ptr(stream))
    if rc != 0:
        raise RuntimeError(f"synth_dev_uniform_int_bf16 failed ({rc})")
