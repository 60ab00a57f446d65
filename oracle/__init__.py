"""CPU oracle of the gradient-bucket reduction: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path never does.

Thin numpy wrappers around ``liboracle.so`` (plain C, see ``oracle.c`` for
the definitions and the passages of the pages they follow). bf16 data is
carried as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIBRARY may name another build of oracle.c (the mutation test loads
# deliberately broken copies through it); by default the in-tree build is used.
LIB = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")

BF16, FP32 = 0, 1
_i32, _i64, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB)
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_bf16.restype = ctypes.c_uint16
        lib.orc_bf16_to_f32_array.argtypes = [_vp, _vp, _i64]
        lib.orc_f32_to_bf16_array.argtypes = [_vp, _vp, _i64]
        lib.orc_ring_run.argtypes = [_i32, _i64, _vp, _i32, _i32, _vp, _i32]
        lib.orc_fold_points.argtypes = [_i32, _i64, _vp, _vp, _vp, _i32]
        lib.orc_exact_sum_points.argtypes = [_i32, _i64, _vp, _vp, _vp]
        lib.orc_reduce_scatter_part.argtypes = [_i32, _i64, _i32, _vp, _i32, _vp, _i32, _i32,
                                                _i64, _i64]
        lib.orc_reduce_scatter.argtypes = [_i32, _i64, _i32, _vp, _i32, _vp, _i32, _i32]
        lib.orc_all_gather.argtypes = [_i32, _i32, _vp, _vp, _vp, _i32, _i32]
        lib.orc_allreduce.argtypes = [_i32, _i64, _i32, _vp, _vp, _i32]
        lib.orc_flatten.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, _i64]
        for f in ("orc_bf16_to_f32_array", "orc_f32_to_bf16_array", "orc_fold_points",
                  "orc_exact_sum_points"):
            getattr(lib, f).restype = None
        for f in ("orc_ring_run", "orc_reduce_scatter_part", "orc_reduce_scatter",
                  "orc_all_gather", "orc_allreduce", "orc_flatten"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return FP32
    raise TypeError(f"unsupported dtype {a.dtype} (bf16 as uint16, or float32)")


def _ptrs(arrays):
    arr = (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return arr


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: invalid arguments")


def chunk_size(N: int, K: int) -> int:
    return -(-N // K)


# ------------------------------------------------------------------- codec
def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    _load().orc_bf16_to_f32_array(h.ctypes.data, out.ctypes.data, h.size)
    return out


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    _load().orc_f32_to_bf16_array(f.ctypes.data, out.ctypes.data, f.size)
    return out


# ------------------------------------------------------------ ring simulator
def ring_run(x: np.ndarray, n_rs: int, n_ag: int = 0, wire: bool = False):
    """x: float32 [K, K*C] per-rank inputs. Runs n_rs scatter-reduce rounds and
    then n_ag all-gather rounds of the literal ring. Returns (state [K, K, C],
    sent [K]) where sent counts the elements each rank put on the wire. With
    wire=True partial sums are rounded to bf16 as they travel."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    K = x.shape[0]
    assert x.shape[1] % K == 0
    C = x.shape[1] // K
    state = x.reshape(K, K, C).copy()
    sent = np.zeros(K, dtype=np.int64)
    _check(_load().orc_ring_run(K, C, state.ctypes.data, n_rs, n_ag, sent.ctypes.data,
                                1 if wire else 0), "ring_run")
    return state, sent


# -------------------------------------------------------------- direct fold
def fold_points(xs: np.ndarray, start: np.ndarray, wire: bool = False) -> np.ndarray:
    """xs float32 [K, n]; start int [n] (rank each point's fold starts at)."""
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    K, n = xs.shape
    st = np.ascontiguousarray(start, dtype=np.int32)
    assert st.shape == (n,) and (n == 0 or (st.min() >= 0 and st.max() < K))
    out = np.empty(n, dtype=np.float32)
    _load().orc_fold_points(K, n, xs.ctypes.data, st.ctypes.data, out.ctypes.data,
                            1 if wire else 0)
    return out


def exact_sum_points(xs: np.ndarray):
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    K, n = xs.shape
    out = np.empty(n, dtype=np.float64)
    ab = np.empty(n, dtype=np.float64)
    _load().orc_exact_sum_points(K, n, xs.ctypes.data, out.ctypes.data, ab.ctypes.data)
    return out, ab


def reduce_scatter(inputs, N, out_dtype, shift=1, average=True, o_range=None, out=None,
                   accumulate=False, wire=False):
    """inputs: list of K arrays (uint16 bf16 or float32) of >= N elements.
    Returns (or fills) K arrays of C = ceil(N/K) elements of out_dtype. With
    accumulate=True, `out` holds the previous partitions and is added into."""
    K = len(inputs)
    C = chunk_size(N, K)
    ins = [np.ascontiguousarray(a) for a in inputs]
    in_dt = _dt(ins[0])
    assert all(_dt(a) == in_dt and a.size >= N for a in ins)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs the previous partitions in `out`")
        out = [np.empty(C, dtype=out_dtype) for _ in range(K)]
    out_dt = _dt(out[0])
    lo, hi = (0, C) if o_range is None else o_range
    flags = (1 if average else 0) | (2 if accumulate else 0) | (4 if wire else 0)
    rc = _load().orc_reduce_scatter_part(K, N, in_dt, _ptrs(ins), out_dt, _ptrs(out), shift,
                                         flags, lo, hi)
    _check(rc, "reduce_scatter")
    return out


def all_gather(shards, fulls, segs, shift):
    """segs: list of (shard_off, full_off, numel); fills `fulls` in place."""
    K = len(shards)
    dt = _dt(shards[0])
    seg_arr = np.ascontiguousarray(np.array(segs, dtype=np.int64).reshape(-1, 3))
    rc = _load().orc_all_gather(K, dt, _ptrs(shards), _ptrs(fulls), seg_arr.ctypes.data,
                                seg_arr.shape[0], shift)
    _check(rc, "all_gather")
    return fulls


def allreduce(inputs, N, average=False, out=None, wire=False):
    K = len(inputs)
    ins = [np.ascontiguousarray(a) for a in inputs]
    dt = _dt(ins[0])
    if out is None:
        out = [np.empty(N, dtype=ins[0].dtype) for _ in range(K)]
    rc = _load().orc_allreduce(K, N, dt, _ptrs(ins), _ptrs(out),
                               (1 if average else 0) | (4 if wire else 0))
    _check(rc, "allreduce")
    return out


def flatten(frags, numels, padded):
    """frags: list over ranks of lists over fragments (same numels on every rank)."""
    K = len(frags)
    F = len(numels)
    flat = [np.ascontiguousarray(f) for row in frags for f in row]
    dt = _dt(flat[0]) if flat else BF16
    dtype = np.uint16 if dt == BF16 else np.float32
    buckets = [np.empty(padded, dtype=dtype) for _ in range(K)]
    nums = np.ascontiguousarray(np.array(numels, dtype=np.int64))
    frag_ptrs = _ptrs(flat) if flat else None
    rc = _load().orc_flatten(K, F, dt, frag_ptrs, nums.ctypes.data if F else None,
                             _ptrs(buckets), padded)
    _check(rc, "flatten")
    return buckets
