"""Python binding of libzr: gradient-bucket reduction on MI355X (gfx950).

Argument marshalling only. Every function here has the name of the C call it
forwards to (see ``include/zr.h`` for the full contract) and does no
arithmetic of its own: it turns per-rank torch tensors into tables of device
pointers, torch streams into ``hipStream_t`` handles, and a non-OK status into
:class:`ZrError`. PyTorch supplies device memory and streams, nothing else.

The library must be built (``__graft_entry__.build()``); importing this module
does not build it, and every call raises if ``libzr.so`` is missing.

Calls (a list holds one buffer per rank, as tensors or integer addresses;
streams default to torch's current stream):

* ``zr_reduce_scatter_avg(inputs, N, outputs, chunk_shift=1, average=True,
  order=ZR_ORDER_RING, accumulate=False)``: ring-order reduce-scatter, /K,
  cast, one write of each rank's partition of ``ceil(N / K)`` elements.
* ``zr_reduce_scatter_frags(frags, numels, N, outputs, ...)``: the same from
  per-parameter fragments, without a bucket; ``RsfPlan(...)`` builds it once
  and ``.launch()`` repeats it.
* ``zr_all_gather(shards, fulls, segs, chunk_shift=0)`` and
  ``zr_allreduce(inputs, outputs, N, average=False, fused=True)``.
* ``zr_flatten_bucket(frags, numels, buckets, padded_numel)``; ``FlatPlan``
  builds it once.
* ``zr_workspace_bytes(K, n)``: the device workspace (a uint8 tensor, or an
  ``(address, bytes)`` pair, passed as ``workspace=``) that lets a call with
  ``n`` fragments or segments go out as one launch.
* ``Sched``: ping-pong bucket buffers with per-buffer completion events
  (``acquire``, ``submit_rs``, ``flush``).
* ``Prefetcher``: ZeRO-3 fetch and prefetch of full parameters into per-rank
  arenas (``fetch``, ``full``, ``release``, ``stats``).
* Host only: ``zr_pf_plan``, ``zr_plan_buckets``, ``zr_cost_*``.

Example: eight ranks' bf16 gradients of N elements reduced into fp32
partitions (rank q receives chunk (q + 1) mod 8, averaged)::

    import torch, gradient_sync_zr_amd as zr
    grads = [torch.randn(N, device="cuda").bfloat16() for _ in range(8)]
    parts = [torch.empty(-(-N // 8), device="cuda") for _ in range(8)]
    zr.zr_reduce_scatter_avg(grads, N, parts)
"""
from __future__ import annotations

import array
import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZR_LIBRARY may name another build of the same library (a different file
# with the same ABI); by default the in-tree build is used.
LIB_PATH = os.environ.get("ZR_LIBRARY") or os.path.join(_HERE, "libzr.so")

(ZR_OK, ZR_ERR_INVALID, ZR_ERR_ALIGN, ZR_ERR_ALIAS, ZR_ERR_UNSUPPORTED, ZR_ERR_WORKSPACE, ZR_ERR_HIP,
 ZR_ERR_NOMEM) = range(8)
ZR_BF16, ZR_FP32 = 0, 1
ZR_ORDER_RING, ZR_ORDER_FREE, ZR_ORDER_RING_WIRE = 0, 1, 2
ZR_AVERAGE, ZR_ACCUMULATE = 1, 2
ZR_MAX_RANKS, ZR_MAX_ELEMS = 64, 1 << 40
ZR_NOALLOC_TABLE_BYTES = 1 << 20
STATUS_NAMES = {0: "ZR_OK", 1: "ZR_ERR_INVALID", 2: "ZR_ERR_ALIGN", 3: "ZR_ERR_ALIAS",
                4: "ZR_ERR_UNSUPPORTED", 5: "ZR_ERR_WORKSPACE", 6: "ZR_ERR_HIP", 7: "ZR_ERR_NOMEM"}

COST_EXPORTS = ("zr_cost_ring_allreduce", "zr_cost_ring_reduce_scatter", "zr_cost_tree_allreduce",
                "zr_cost_naive_allreduce", "zr_cost_pipelined_broadcast",
                "zr_cost_best_broadcast_segments", "zr_cost_ring_tree_crossover",
                "zr_cost_ring_naive_crossover", "zr_cost_dp_speedup")
RS_PLAN_EXPORTS = ("zr_rs_plan_create", "zr_rs_plan_launch", "zr_rs_plan_destroy")
RSF_PLAN_EXPORTS = ("zr_rsf_plan_create", "zr_rsf_plan_launch", "zr_rsf_plan_info", "zr_rsf_plan_destroy")
FLAT_PLAN_EXPORTS = ("zr_flatten_plan_create", "zr_flatten_plan_launch", "zr_flatten_plan_info",
                     "zr_flatten_plan_destroy")
PF_EXPORTS = ("zr_pf_create", "zr_pf_fetch", "zr_pf_release", "zr_pf_full", "zr_pf_get_stats",
              "zr_pf_destroy", "zr_pf_plan")
EXPORTS = ("zr_last_error", "zr_version", "zr_workspace_bytes", "zr_flatten_bucket", "zr_reduce_scatter_avg",
           "zr_reduce_scatter_frags", "zr_all_gather", "zr_allreduce", "zr_plan_buckets", "zr_sched_create",
           "zr_sched_acquire", "zr_sched_submit_rs", "zr_sched_flush",
           "zr_sched_destroy", "zr_reduce_scatter_frags_noalloc") + COST_EXPORTS + PF_EXPORTS + \
    RSF_PLAN_EXPORTS + FLAT_PLAN_EXPORTS + RS_PLAN_EXPORTS


class ZrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class zr_seg(ctypes.Structure):
    _fields_ = [("shard_off", ctypes.c_int64), ("full_off", ctypes.c_int64),
                ("numel", ctypes.c_int64)]


class zr_pf_config(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int), ("dtype", ctypes.c_int), ("n_params", ctypes.c_int),
                ("numels", ctypes.POINTER(ctypes.c_int64)),
                ("shard_offsets", ctypes.POINTER(ctypes.c_int64)),
                ("shards", ctypes.POINTER(ctypes.c_void_p)),
                ("arenas", ctypes.POINTER(ctypes.c_void_p)),
                ("arena_numel", ctypes.c_int64), ("chunk_shift", ctypes.c_int),
                ("n_steps", ctypes.c_int), ("step_offsets", ctypes.POINTER(ctypes.c_int32)),
                ("step_params", ctypes.POINTER(ctypes.c_int32)),
                ("prefetch_bucket_numel", ctypes.c_int64), ("max_live_numel", ctypes.c_int64),
                ("max_reuse_numel", ctypes.c_int64),
                ("max_ongoing_fetches", ctypes.c_int), ("gather_stream", ctypes.c_void_p),
                ("compute_stream", ctypes.c_void_p)]


PF_STAT_FIELDS = ("gathers", "immediate_gathers", "immediate_numel", "prefetch_numel", "host_syncs",
                  "stream_waits", "live", "peak_live", "peak_ongoing", "arena_peak",
                  "prefetch_trimmed", "retained")


class zr_pf_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in PF_STAT_FIELDS]


_lib = None
_i32, _i64, _vp, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
_PP = ctypes.POINTER(ctypes.c_void_p)


def lib() -> ctypes.CDLL:
    """The loaded libzr (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: the HIP library is not built "
                               "(run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.zr_last_error.restype = ctypes.c_char_p
        L.zr_version.restype = ctypes.c_int
        L.zr_workspace_bytes.argtypes = [_i32, _i32]
        L.zr_workspace_bytes.restype = _sz
        L.zr_flatten_bucket.argtypes = [_i32, _i32, _PP, ctypes.POINTER(_i64), _PP, _i64, _i32, _vp, _sz, _vp]
        L.zr_reduce_scatter_avg.argtypes = [_i32, _PP, _i32, _i64, _PP, _i32, _i32, _i32, _i32, _vp]
        L.zr_all_gather.argtypes = [_i32, _PP, _PP, _i32, ctypes.POINTER(zr_seg), _i32, _i32, _vp, _sz,
                                    _vp]
        L.zr_reduce_scatter_frags.argtypes = [_i32, _i32, _PP, ctypes.POINTER(_i64), _i64, _i32, _PP,
                                              _i32, _i32, _i32, _i32, _vp, _sz, _vp]
        L.zr_reduce_scatter_frags_noalloc.argtypes = [_i32, _i32, _PP, ctypes.POINTER(_i64), _i64, _i32,
                                                      _PP, _i32, _i32, _i32, _i32, _vp]
        L.zr_allreduce.argtypes = [_i32, _PP, _PP, _i32, _i64, _i32, _i32, _i32, _vp, _vp]
        L.zr_plan_buckets.argtypes = [_i32, ctypes.POINTER(_i64), _i64, ctypes.POINTER(ctypes.c_int32),
                                      ctypes.POINTER(ctypes.c_int32)]
        L.zr_sched_create.argtypes = [ctypes.POINTER(_vp), _i32, _i32, _vp]
        L.zr_sched_acquire.argtypes = [_vp, _i32, _vp]
        L.zr_sched_submit_rs.argtypes = [_vp, _i32, _PP, _i32, _i32, _PP, _i32, _i64, _PP, _i32,
                                         _i32, _i32, _i32]
        L.zr_sched_flush.argtypes = [_vp, _vp]
        L.zr_sched_destroy.argtypes = [_vp]
        L.zr_rsf_plan_create.argtypes = [_i32, _i32, _PP, ctypes.POINTER(_i64), _i64, _i32, _PP, _i32,
                                         _i32, _i32, _i32, _vp, _sz, ctypes.POINTER(_vp)]
        L.zr_rs_plan_create.argtypes = [_i32, _PP, _i32, _i64, _PP, _i32, _i32, _i32, _i32,
                                        ctypes.POINTER(_vp)]
        L.zr_rs_plan_launch.argtypes = [_vp, _vp]
        L.zr_rs_plan_destroy.argtypes = [_vp]
        L.zr_rsf_plan_launch.argtypes = [_vp, _vp]
        L.zr_rsf_plan_info.argtypes = [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_sz)]
        L.zr_rsf_plan_destroy.argtypes = [_vp]
        L.zr_flatten_plan_create.argtypes = [_i32, _i32, _PP, ctypes.POINTER(_i64), _PP, _i64, _i32, _vp,
                                             _sz, ctypes.POINTER(_vp)]
        L.zr_flatten_plan_launch.argtypes = [_vp, _vp]
        L.zr_flatten_plan_info.argtypes = [_vp, ctypes.POINTER(_i32), ctypes.POINTER(_sz)]
        L.zr_flatten_plan_destroy.argtypes = [_vp]
        _cfgp = ctypes.POINTER(zr_pf_config)
        L.zr_pf_create.argtypes = [_cfgp, ctypes.POINTER(_vp)]
        L.zr_pf_fetch.argtypes = [_vp, _i32]
        L.zr_pf_release.argtypes = [_vp, _i32]
        L.zr_pf_full.argtypes = [_vp, _i32, _i32, ctypes.POINTER(_vp)]
        L.zr_pf_get_stats.argtypes = [_vp, ctypes.POINTER(zr_pf_stats)]
        L.zr_pf_destroy.argtypes = [_vp]
        L.zr_pf_plan.argtypes = [_cfgp, _i32, ctypes.POINTER(zr_pf_stats)]
        for f in EXPORTS[3:]:
            getattr(L, f).restype = ctypes.c_int
        _d = ctypes.c_double
        for f in ("zr_cost_ring_allreduce", "zr_cost_ring_reduce_scatter",
                  "zr_cost_tree_allreduce", "zr_cost_naive_allreduce"):
            getattr(L, f).argtypes = [_i32, _d, _d, _d]
            getattr(L, f).restype = _d
        L.zr_cost_pipelined_broadcast.argtypes = [_i32, _d, _i32, _d, _d]
        L.zr_cost_pipelined_broadcast.restype = _d
        L.zr_cost_best_broadcast_segments.argtypes = [_i32, _d, _d, _d, _i32,
                                                      ctypes.POINTER(_d)]
        L.zr_cost_best_broadcast_segments.restype = _i32
        for f in ("zr_cost_ring_tree_crossover", "zr_cost_ring_naive_crossover"):
            getattr(L, f).argtypes = [_i32, _d, _d]
            getattr(L, f).restype = _d
        L.zr_cost_dp_speedup.argtypes = [_i32, _d, _d, _d, _d]
        L.zr_cost_dp_speedup.restype = _d
        _lib = L
    return _lib


def _check(status: int):
    if status != ZR_OK:
        raise ZrError(status, lib().zr_last_error().decode(errors="replace"))


# ------------------------------------------------------------ marshalling
def _ptr(x) -> int:
    """Device address of a tensor, or an int address passed through."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _table(xs: Optional[Sequence]):
    """A C array of device addresses (void*[]), built through array.array: for
    hundreds of fragment pointers this is several times cheaper than filling
    a ctypes array element by element. A table built once with ``table()``
    passes through unchanged."""
    if xs is None:
        return None
    if isinstance(xs, ctypes.Array):
        return xs  # already a table (a caller that reuses one across calls)
    try:
        a = array.array("Q", xs or [0])  # a list of int addresses
    except TypeError:
        a = array.array("Q", [_ptr(x) for x in xs])
    t = (ctypes.c_void_p * len(a)).from_buffer(a)
    t._keep = a  # the array owns the memory the C array views
    return t


def table(xs: Sequence):
    """A reusable C table of device addresses for the per-rank arguments."""
    return _table(xs)


def _int64s(xs: Sequence[int]):
    """A C array of int64 (sizes), built through array.array."""
    a = array.array("q", list(xs) or [0])
    t = (ctypes.c_int64 * len(a)).from_buffer(a)
    t._keep = a
    return t


def _dtype(x) -> int:
    import torch
    if isinstance(x, int):
        return x
    dt = x if isinstance(x, torch.dtype) else x.dtype
    if dt == torch.bfloat16:
        return ZR_BF16
    if dt == torch.float32:
        return ZR_FP32
    raise TypeError(f"unsupported dtype {dt}: bfloat16 or float32")


def _workspace(ws):
    """(device address, bytes) of a workspace: None, a tensor, or a pair."""
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws[0], ws[1]
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _stream(stream) -> int:
    """hipStream_t of a torch stream (None = torch's current stream)."""
    if isinstance(stream, int):
        return stream
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ------------------------------------------------------------------- calls
def zr_version() -> int:
    return lib().zr_version()


def zr_last_error() -> str:
    return lib().zr_last_error().decode(errors="replace")


def zr_workspace_bytes(K: int, n: int) -> int:
    return lib().zr_workspace_bytes(K, n)


def zr_flatten_bucket(frags: Sequence[Sequence], numels: Sequence[int], buckets: Sequence,
                      padded_numel: int, dtype=None, stream=None, workspace=None) -> None:
    """frags[r][p] = fragment p of rank r; buckets[r] = rank r's flat bucket."""
    K = len(buckets)
    F = len(numels)
    flat = [f for row in frags for f in row]
    if len(flat) != K * F:
        raise ValueError("frags must be K lists of len(numels) tensors")
    dt = _dtype(dtype if dtype is not None else buckets[0])
    nums = _int64s(numels)
    ws, wsb = _workspace(workspace)
    _check(lib().zr_flatten_bucket(K, F, _table(flat), nums, _table(buckets), padded_numel, dt, ws, wsb,
                                   _stream(stream)))


class FlatPlan:
    """zr_flatten_plan_*: a bucket flatten validated and built once (its table
    staged in `workspace` when it needs one); launch() enqueues it."""

    def __init__(self, frags: Sequence[Sequence], numels: Sequence[int], buckets: Sequence,
                 padded_numel: int, dtype=None, workspace=None):
        K = len(buckets)
        F = len(numels)
        flat = [f for row in frags for f in row]
        if len(flat) != K * F:
            raise ValueError("frags must be K lists of len(numels) tensors")
        dt = _dtype(dtype if dtype is not None else buckets[0])
        ws, wsb = _workspace(workspace)
        h = ctypes.c_void_p()
        _check(lib().zr_flatten_plan_create(K, F, _table(flat), _int64s(numels), _table(buckets),
                                            padded_numel, dt, ws, wsb, ctypes.byref(h)))
        self._h = h
        self.workspace = workspace  # used by every launch

    def launch(self, stream=None) -> None:
        _check(lib().zr_flatten_plan_launch(self._h, _stream(stream)))

    def info(self) -> dict:
        n, b = ctypes.c_int(0), ctypes.c_size_t(0)
        _check(lib().zr_flatten_plan_info(self._h, ctypes.byref(n), ctypes.byref(b)))
        return {"launches": n.value, "table_bytes": b.value}

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().zr_flatten_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _flags(average: bool, accumulate: bool) -> int:
    return (ZR_AVERAGE if average else 0) | (ZR_ACCUMULATE if accumulate else 0)


def zr_reduce_scatter_avg(inputs: Sequence, N: int, outputs: Sequence, chunk_shift: int = 1,
                          average: bool = True, order: int = ZR_ORDER_RING, in_dtype=None,
                          out_dtype=None, stream=None, accumulate: bool = False) -> None:
    K = len(inputs)
    in_dt = _dtype(in_dtype if in_dtype is not None else inputs[0])
    out_dt = _dtype(out_dtype if out_dtype is not None else outputs[0])
    _check(lib().zr_reduce_scatter_avg(K, _table(inputs), in_dt, N, _table(outputs), out_dt,
                                       chunk_shift, _flags(average, accumulate), order,
                                       _stream(stream)))


class RsPlan:
    """zr_rs_plan_*: a reduce-scatter validated and built once; launch()
    enqueues it on a stream (torch's current one by default)."""

    def __init__(self, inputs: Sequence, N: int, outputs: Sequence, chunk_shift: int = 1,
                 average: bool = True, order: int = ZR_ORDER_RING, in_dtype=None, out_dtype=None,
                 accumulate: bool = False):
        K = len(inputs)
        in_dt = _dtype(in_dtype if in_dtype is not None else inputs[0])
        out_dt = _dtype(out_dtype if out_dtype is not None else outputs[0])
        h = ctypes.c_void_p()
        _check(lib().zr_rs_plan_create(K, _table(inputs), in_dt, N, _table(outputs), out_dt, chunk_shift,
                                       _flags(average, accumulate), order, ctypes.byref(h)))
        self._h = h

    def launch(self, stream=None) -> None:
        _check(lib().zr_rs_plan_launch(self._h, _stream(stream)))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().zr_rs_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def zr_reduce_scatter_frags(frags: Sequence[Sequence], numels: Sequence[int], N: int,
                            outputs: Sequence, chunk_shift: int = 1, average: bool = True,
                            order: int = ZR_ORDER_RING, in_dtype=None, out_dtype=None,
                            stream=None, accumulate: bool = False, workspace=None) -> None:
    """frags[r][p] = fragment p of rank r (same numels on every rank)."""
    K = len(outputs)
    F = len(numels)
    flat = [f for row in frags for f in row]
    if len(flat) != K * F:
        raise ValueError("frags must be K lists of len(numels) tensors")
    in_dt = _dtype(in_dtype if in_dtype is not None else flat[0])
    out_dt = _dtype(out_dtype if out_dtype is not None else outputs[0])
    nums = _int64s(numels)
    ws, wsb = _workspace(workspace)
    _check(lib().zr_reduce_scatter_frags(K, F, _table(flat), nums, N, in_dt, _table(outputs),
                                         out_dt, chunk_shift, _flags(average, accumulate), order,
                                         ws, wsb, _stream(stream)))


def zr_reduce_scatter_frags_noalloc(frags: Sequence[Sequence], numels: Sequence[int], N: int,
                                    outputs: Sequence, chunk_shift: int = 1, average: bool = True,
                                    order: int = ZR_ORDER_RING, in_dtype=None, out_dtype=None,
                                    stream=None, accumulate: bool = False) -> None:
    """zr_reduce_scatter_frags staging its table in the library's own device
    array (no workspace, nothing allocated)."""
    K = len(outputs)
    F = len(numels)
    flat = [f for row in frags for f in row]
    if len(flat) != K * F:
        raise ValueError("frags must be K lists of len(numels) tensors")
    in_dt = _dtype(in_dtype if in_dtype is not None else flat[0])
    out_dt = _dtype(out_dtype if out_dtype is not None else outputs[0])
    _check(lib().zr_reduce_scatter_frags_noalloc(K, F, _table(flat), _int64s(numels), N, in_dt,
                                                 _table(outputs), out_dt, chunk_shift,
                                                 _flags(average, accumulate), order, _stream(stream)))


class RsfPlan:
    """zr_rsf_plan_*: a discrete reduce-scatter validated and built once;
    launch() enqueues it on a stream (torch's current one by default)."""

    def __init__(self, frags: Sequence[Sequence], numels: Sequence[int], N: int, outputs: Sequence,
                 chunk_shift: int = 1, average: bool = True, order: int = ZR_ORDER_RING,
                 in_dtype=None, out_dtype=None, accumulate: bool = False, workspace=None):
        K = len(outputs)
        F = len(numels)
        flat = [f for row in frags for f in row]
        if len(flat) != K * F:
            raise ValueError("frags must be K lists of len(numels) tensors")
        in_dt = _dtype(in_dtype if in_dtype is not None else flat[0])
        out_dt = _dtype(out_dtype if out_dtype is not None else outputs[0])
        ws, wsb = _workspace(workspace)
        h = ctypes.c_void_p()
        _check(lib().zr_rsf_plan_create(K, F, _table(flat), _int64s(numels), N, in_dt,
                                        _table(outputs), out_dt, chunk_shift,
                                        _flags(average, accumulate), order, ws, wsb,
                                        ctypes.byref(h)))
        self._h = h
        self.workspace = workspace  # used by every launch

    def launch(self, stream=None) -> None:
        _check(lib().zr_rsf_plan_launch(self._h, _stream(stream)))

    def info(self) -> dict:
        n, b = ctypes.c_int(0), ctypes.c_size_t(0)
        _check(lib().zr_rsf_plan_info(self._h, ctypes.byref(n), ctypes.byref(b)))
        return {"launches": n.value, "table_bytes": b.value}

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().zr_rsf_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def zr_all_gather(shards: Sequence, fulls: Sequence, segs: Sequence, chunk_shift: int = 0,
                  dtype=None, stream=None, workspace=None) -> None:
    """segs: (shard_off, full_off, numel) triples."""
    K = len(shards)
    dt = _dtype(dtype if dtype is not None else shards[0])
    arr = (zr_seg * max(1, len(segs)))(*[zr_seg(*s) for s in segs])
    ws, wsb = _workspace(workspace)
    _check(lib().zr_all_gather(K, _table(shards), _table(fulls), dt, arr, len(segs), chunk_shift,
                               ws, wsb, _stream(stream)))


def zr_allreduce(inputs: Sequence, outputs: Sequence, N: int, average: bool = False,
                 order: int = ZR_ORDER_RING, fused: bool = True, scratch=None, dtype=None,
                 stream=None) -> None:
    K = len(inputs)
    dt = _dtype(dtype if dtype is not None else inputs[0])
    _check(lib().zr_allreduce(K, _table(inputs), _table(outputs), dt, N, 1 if average else 0,
                              order, 1 if fused else 0, _ptr(scratch), _stream(stream)))


def zr_plan_buckets(numels: Sequence[int], cap: int):
    """Returns (bucket_of list, n_buckets)."""
    n = len(numels)
    arr = _int64s(numels)
    out = (ctypes.c_int32 * max(1, n))()
    nb = ctypes.c_int32(0)
    _check(lib().zr_plan_buckets(n, arr, cap, out, ctypes.byref(nb)))
    return list(out)[:n], nb.value


# ------------------------------------------------------------- cost model
def zr_cost_ring_allreduce(K, nbytes, alpha, beta):
    return lib().zr_cost_ring_allreduce(K, nbytes, alpha, beta)


def zr_cost_ring_reduce_scatter(K, nbytes, alpha, beta):
    return lib().zr_cost_ring_reduce_scatter(K, nbytes, alpha, beta)


def zr_cost_tree_allreduce(K, nbytes, alpha, beta):
    return lib().zr_cost_tree_allreduce(K, nbytes, alpha, beta)


def zr_cost_naive_allreduce(K, nbytes, alpha, beta):
    return lib().zr_cost_naive_allreduce(K, nbytes, alpha, beta)


def zr_cost_pipelined_broadcast(K, nbytes, segments, alpha, beta):
    return lib().zr_cost_pipelined_broadcast(K, nbytes, segments, alpha, beta)


def zr_cost_best_broadcast_segments(K, nbytes, alpha, beta, max_segments=1 << 20):
    """Returns (segments, time)."""
    t = ctypes.c_double(0.0)
    s = lib().zr_cost_best_broadcast_segments(K, nbytes, alpha, beta, max_segments,
                                              ctypes.byref(t))
    return s, t.value


def zr_cost_ring_tree_crossover(K, alpha, beta):
    return lib().zr_cost_ring_tree_crossover(K, alpha, beta)


def zr_cost_ring_naive_crossover(K, alpha, beta):
    return lib().zr_cost_ring_naive_crossover(K, alpha, beta)


def zr_cost_dp_speedup(K, t1, grad_bytes, alpha, beta):
    return lib().zr_cost_dp_speedup(K, t1, grad_bytes, alpha, beta)


class Sched:
    """zr_sched_*: ping-pong IPG buffers with per-buffer completion events."""

    def __init__(self, n_buffers: int = 2, max_producers: int = 4, reduction_stream=None):
        h = ctypes.c_void_p()
        self.reduction_stream = reduction_stream
        _check(lib().zr_sched_create(ctypes.byref(h), n_buffers, max_producers,
                                     _stream(reduction_stream)))
        self._h = h

    def acquire(self, buf: int, producer_stream=None) -> None:
        _check(lib().zr_sched_acquire(self._h, buf, _stream(producer_stream)))

    def submit_rs(self, buf: int, producer_streams: Sequence, inputs: Sequence, N: int,
                  outputs: Sequence, chunk_shift: int = 1, average: bool = True,
                  order: int = ZR_ORDER_RING, in_dtype=None, out_dtype=None,
                  accumulate: bool = False) -> None:
        K = len(inputs)
        prods = (ctypes.c_void_p * max(1, len(producer_streams)))(
            *[_stream(p) for p in producer_streams])
        in_dt = _dtype(in_dtype if in_dtype is not None else inputs[0])
        out_dt = _dtype(out_dtype if out_dtype is not None else outputs[0])
        _check(lib().zr_sched_submit_rs(self._h, buf, prods, len(producer_streams), K,
                                        _table(inputs), in_dt, N, _table(outputs), out_dt,
                                        chunk_shift, _flags(average, accumulate), order))

    def flush(self, caller_stream=None) -> None:
        _check(lib().zr_sched_flush(self._h, _stream(caller_stream)))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().zr_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------- prefetch coordinator
def _pf_config(K, dtype, numels, steps, prefetch_bucket_numel, max_live_numel, arena_numel,
               max_ongoing_fetches=2, max_reuse_numel=0, shard_offsets=None, shards=None,
               arenas=None, chunk_shift=0, gather_stream=None, compute_stream=None):
    """zr_pf_config plus the arrays it points to (kept alive with it).
    steps: one list of parameter ids per step, in trace order."""
    offs, flat = [0], []
    for st in steps:
        flat.extend(int(p) for p in st)
        offs.append(len(flat))
    keep = {
        "numels": _int64s(numels),
        "step_offsets": (ctypes.c_int32 * len(offs))(*offs),
        "step_params": (ctypes.c_int32 * max(1, len(flat)))(*flat),
    }
    c = zr_pf_config()
    c.K, c.dtype, c.n_params = K, _dtype(dtype), len(numels)
    c.numels = keep["numels"]
    if shard_offsets is not None:
        keep["shard_offsets"] = _int64s(shard_offsets)
        c.shard_offsets = keep["shard_offsets"]
    if shards is not None:
        keep["shards"] = _table(shards)
        c.shards = keep["shards"]
    if arenas is not None:
        keep["arenas"] = _table(arenas)
        c.arenas = keep["arenas"]
    c.arena_numel, c.chunk_shift = arena_numel, chunk_shift
    c.n_steps = len(steps)
    c.step_offsets, c.step_params = keep["step_offsets"], keep["step_params"]
    c.prefetch_bucket_numel, c.max_live_numel = prefetch_bucket_numel, max_live_numel
    c.max_reuse_numel = max_reuse_numel
    c.max_ongoing_fetches = max_ongoing_fetches
    c.gather_stream = _stream(gather_stream) if gather_stream is not None or shards is not None else None
    c.compute_stream = _stream(compute_stream) if compute_stream is not None or shards is not None else None
    c._keep = keep
    return c


def _stats_dict(st: zr_pf_stats) -> dict:
    return {n: getattr(st, n) for n in PF_STAT_FIELDS}


def zr_pf_plan(numels: Sequence[int], steps: Sequence[Sequence[int]], prefetch_bucket_numel: int,
               max_live_numel: int, arena_numel: int, max_ongoing_fetches: int = 2,
               max_reuse_numel: int = 0, iterations: int = 1, K: int = 8, dtype=ZR_BF16) -> dict:
    """Host-only run of the trace (gathers finish at once): the counters a
    coordinator with this config reaches, e.g. peak live elements and the
    arena peak, to size an arena."""
    c = _pf_config(K, dtype, numels, steps, prefetch_bucket_numel, max_live_numel, arena_numel,
                   max_ongoing_fetches, max_reuse_numel)
    st = zr_pf_stats()
    _check(lib().zr_pf_plan(ctypes.byref(c), iterations, ctypes.byref(st)))
    return _stats_dict(st)


class Prefetcher:
    """zr_pf_*: ZeRO-3 fetch / prefetch of full parameters into per-rank
    arenas, gathers on `gather_stream`, consumers on `compute_stream`."""

    def __init__(self, numels: Sequence[int], shard_offsets: Sequence[int], shards: Sequence,
                 arenas: Sequence, arena_numel: int, steps: Sequence[Sequence[int]],
                 prefetch_bucket_numel: int, max_live_numel: int, max_ongoing_fetches: int = 2,
                 max_reuse_numel: int = 0, chunk_shift: int = 0, gather_stream=None,
                 compute_stream=None, dtype=None):
        self.K = len(shards)
        self.n_steps = len(steps)
        dt = dtype if dtype is not None else shards[0]
        self._cfg = _pf_config(self.K, dt, numels, steps, prefetch_bucket_numel, max_live_numel,
                               arena_numel, max_ongoing_fetches, max_reuse_numel, shard_offsets,
                               shards, arenas, chunk_shift, gather_stream, compute_stream)
        h = ctypes.c_void_p()
        _check(lib().zr_pf_create(ctypes.byref(self._cfg), ctypes.byref(h)))
        self._h = h

    def fetch(self, step: int) -> None:
        _check(lib().zr_pf_fetch(self._h, step))

    def release(self, step: int) -> None:
        _check(lib().zr_pf_release(self._h, step))

    def full(self, param: int, rank: int) -> int:
        """Device address of a live parameter's full copy on `rank`."""
        p = ctypes.c_void_p()
        _check(lib().zr_pf_full(self._h, param, rank, ctypes.byref(p)))
        return p.value

    def stats(self) -> dict:
        st = zr_pf_stats()
        _check(lib().zr_pf_get_stats(self._h, ctypes.byref(st)))
        return _stats_dict(st)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().zr_pf_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
