"""GPU parity on IEEE special values.

The values are subnormals, signed zeros, values near the largest finite, infinities and NaNs. They go
through every entry point that does arithmetic:
  - the reduce-scatter, in every dtype pair and in both ring orders, with averaging by a power of two
    and by 5 (the IEEE divide), and with accumulation;
  - the fused and composed all-reduce;
  - the discrete path.
They also go through the two bitwise copies, the all-gather and the flatten.

Readings:
  - The fp32 adds, the average and the bf16 rounding keep subnormals on both sides; nothing is flushed
    to zero.
  - Signed zeros follow IEEE 754.
  - A NaN result is compared only as a NaN. IEEE 754 fixes neither its sign nor its payload, and x86
    and the GPU pick different ones: x86 gives a negative quiet NaN for inf - inf.
  - Every other output is compared bit for bit.
  - The copies move bits, so they keep every NaN payload, signalling ones included.
"""
import numpy as np
import pytest

import oracle
from gpu_util import Guarded, bits

pytestmark = pytest.mark.gpu

RING, WIRE = 0, 2


def zr():
    import gradient_sync_zr_amd as m
    return m


def torch_dt(is_bf16):
    import torch
    return torch.bfloat16 if is_bf16 else torch.float32


def special(rng, K, N, fp32):
    """K arrays of N raw patterns (uint16 bf16, or float32 viewed from uint32).

    Each index draws one scenario, shared by all ranks:
      0  subnormals;
      1  signed zeros: -0 on every rank at half the indices, random signs elsewhere;
      2  the largest finite magnitudes, whose sums overflow or cancel;
      3  +-inf on about 30% of the ranks, normals elsewhere;
      4  a NaN on one rank (quiet, signalling, negative, all ones), normals elsewhere;
      5  normals of mixed sign;
      6  (fp32 only) one rank holds a normal with random low bits, ties to bf16 included, the others
         hold +0; averaging leaves the mantissa unchanged, so the bf16 rounding of that exact value is
         what the output shows.
    """
    scen = rng.integers(0, 7 if fp32 else 6, N)
    neg_all = rng.random(N) < 0.5  # zeros: every rank -0 at half the indices
    if fp32:
        sign = (rng.random((K, N)) < 0.5).astype(np.uint32) << 31
        sub = sign | rng.integers(1, 1 << 23, (K, N), dtype=np.uint32)
        zer = np.where(neg_all | (rng.random((K, N)) < 0.5), 0x80000000, 0).astype(np.uint32)
        big = sign | (0x7F7FFFFE + rng.integers(0, 2, (K, N), dtype=np.uint32))
        nrm = sign | rng.integers(0x3F000000, 0x41000000, (K, N), dtype=np.uint32)
        inf = np.where(rng.random((K, N)) < 0.3, sign | 0x7F800000, nrm).astype(np.uint32)
        nanpat = np.array([0x7FC00000, 0x7F800001, 0xFFC00001, 0xFFFFFFFF], dtype=np.uint32)
        one = np.zeros((K, N), dtype=np.uint32)
        low = rng.integers(0, 1 << 16, N, dtype=np.uint32)
        low = np.where(rng.random(N) < 0.3, 0x8000, low).astype(np.uint32)  # exact ties
        hi = rng.integers(0x3F00, 0x7F80, N, dtype=np.uint32)
        hi = np.where(rng.random(N) < 0.1, 0x7F7F, hi).astype(np.uint32)   # next to the bf16 max
        one[rng.integers(0, K, N), np.arange(N)] = (sign[0] | (hi << 16) | low)
        out = np.empty((K, N), dtype=np.uint32)
    else:
        sign = (rng.random((K, N)) < 0.5).astype(np.uint16) << 15
        sub = sign | rng.integers(0, 128, (K, N), dtype=np.uint16)
        zer = np.where(neg_all | (rng.random((K, N)) < 0.5), 0x8000, 0).astype(np.uint16)
        big = sign | (0x7F7E + rng.integers(0, 2, (K, N), dtype=np.uint16))
        nrm = sign | rng.integers(0x3F00, 0x4100, (K, N), dtype=np.uint16)
        inf = np.where(rng.random((K, N)) < 0.3, sign | 0x7F80, nrm).astype(np.uint16)
        nanpat = np.array([0x7FC0, 0x7F81, 0xFFC1, 0xFFFF], dtype=np.uint16)
        one = None
        out = np.empty((K, N), dtype=np.uint16)
    nan = nrm.copy()
    nan[rng.integers(0, K, N), np.arange(N)] = nanpat[rng.integers(0, 4, N)]
    arrays = [sub, zer, big, inf, nan, nrm] + ([one] if fp32 else [])
    for s, arr in enumerate(arrays):
        out[:, scen == s] = arr[:, scen == s]
    if fp32:
        return [out[r].view(np.float32) for r in range(K)]
    return [out[r] for r in range(K)]


def is_nan(a: np.ndarray) -> np.ndarray:
    b = bits(a)
    if a.dtype == np.float32:
        return (b & 0x7FFFFFFF) > 0x7F800000
    return (b & 0x7FFF) > 0x7F80


def classes(a: np.ndarray):
    """Counts of the special results in an output: subnormal, -0, inf, NaN."""
    b = bits(a).astype(np.int64)
    if a.dtype == np.float32:
        mag, expo, sgn = b & 0x7FFFFFFF, (b >> 23) & 0xFF, b >> 31
        inf_pat = 0x7F800000
    else:
        mag, expo, sgn = b & 0x7FFF, (b >> 7) & 0xFF, b >> 15
        inf_pat = 0x7F80
    return {"subnormal": int(np.sum((expo == 0) & (mag != 0))),
            "neg_zero": int(np.sum((mag == 0) & (sgn == 1))),
            "inf": int(np.sum(mag == inf_pat)),
            "nan": int(np.sum(is_nan(a)))}


def assert_match(got: np.ndarray, want: np.ndarray, what: str):
    wn, gn = is_nan(want), is_nan(got)
    assert np.array_equal(wn, gn), f"{what}: NaN positions differ ({int(np.sum(wn != gn))} of {wn.size})"
    diff = bits(got)[~wn] != bits(want)[~wn]
    assert not diff.any(), f"{what}: {int(np.sum(diff))} of {int(np.sum(~wn))} non-NaN outputs differ"


SMALL = None        # K * 2048 * 3 + 37 * K + 5: a few tiles, one slice per wave
FOUR = 8 * 300000 + 13  # enough tiles for the four-slice tiles of large buckets

RS_CASES = [
    # K, N, in_bf16, out_bf16, average, order, offset, accumulate
    (8, SMALL, True, False, True, RING, 0, False),
    (8, SMALL, True, True, True, RING, 0, False),
    (8, SMALL, False, False, True, RING, 0, False),
    (8, SMALL, False, True, False, RING, 0, False),   # bf16 rounding of exact sums, overflow ties
    (8, SMALL, False, True, True, RING, 0, False),
    (5, SMALL, True, False, True, RING, 0, False),    # IEEE divide of subnormal sums
    (5, SMALL, False, False, True, RING, 0, False),
    (8, SMALL, True, False, True, RING, 1, False),    # element-wise path
    (8, SMALL, True, False, True, WIRE, 0, False),
    (5, SMALL, True, True, True, WIRE, 0, False),
    (8, SMALL, True, False, True, RING, 0, True),     # accumulate into special partitions
    (8, SMALL, False, False, False, RING, 1, True),
    (64, SMALL, True, False, True, RING, 0, False),   # generic-K fold
    (8, FOUR, True, False, True, RING, 0, False),     # the large-bucket kernel
    (8, FOUR, True, False, True, RING, 0, True),
    (8, FOUR, True, True, True, WIRE, 0, False),
]


@pytest.mark.parametrize("K,N,in_bf16,out_bf16,average,order,offset,acc", RS_CASES)
def test_reduce_scatter_special_values(K, N, in_bf16, out_bf16, average, order, offset, acc):
    import torch
    N = N or K * 2048 * 3 + 37 * K + 5
    C = -(-N // K)
    rng = np.random.default_rng(K * 131 + N + 7 * order + offset + (3 if acc else 0))
    xs = special(rng, K, N, fp32=not in_bf16)
    odt = np.uint16 if out_bf16 else np.float32
    if acc:
        olds = special(rng, K, C, fp32=not out_bf16)
    else:
        olds = [np.zeros(C, dtype=odt) for _ in range(K)]
    ins = [Guarded(N, torch_dt(in_bf16), offset, xs[r]) for r in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), offset, olds[r]) for r in range(K)]
    zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs], chunk_shift=1,
                               average=average, order=order, in_dtype=torch_dt(in_bf16),
                               out_dtype=torch_dt(out_bf16), accumulate=acc)
    torch.cuda.synchronize()
    want = [o.copy() for o in olds]
    oracle.reduce_scatter(xs, N, odt, shift=1, average=average, out=want, accumulate=acc,
                          wire=(order == WIRE))
    seen = {"subnormal": 0, "neg_zero": 0, "inf": 0, "nan": 0}
    for r in range(K):
        assert_match(outs[r].get(), want[r], f"rank {r}")
        assert outs[r].guards_intact() and ins[r].guards_intact()
        for k, v in classes(want[r]).items():
            seen[k] += v
    # the case really exercises every class of special result
    assert all(v > 0 for v in seen.values()), seen


@pytest.mark.parametrize("K,bf16,average,order,fused", [
    (8, True, False, RING, True),
    (5, False, True, RING, True),
    (8, True, True, WIRE, True),
    (64, True, False, RING, True),
    (8, True, True, RING, False),    # composed: reduce-scatter, then all-gather
])
def test_allreduce_special_values(K, bf16, average, order, fused):
    import torch
    N = K * 4096 * 2 + 77
    C = -(-N // K)
    rng = np.random.default_rng(K * 17 + N + order + (5 if fused else 0))
    xs = special(rng, K, N, fp32=not bf16)
    bufs = [Guarded(N, torch_dt(bf16), 0, xs[r]) for r in range(K)]
    scratch = None if fused else torch.empty(K * C, dtype=torch_dt(bf16), device="cuda")
    zr().zr_allreduce([g.ptr() for g in bufs], [g.ptr() for g in bufs], N, average=average,
                      order=order, fused=fused, scratch=scratch, dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    want = oracle.allreduce(xs, N, average=average, wire=(order == WIRE))
    got0 = bufs[0].get()
    assert_match(got0, want[0], "rank 0")
    seen = classes(want[0])
    assert all(v > 0 for v in seen.values()), seen
    for r in range(1, K):
        assert np.array_equal(bits(bufs[r].get()), bits(got0)), f"rank {r} differs from rank 0"
        assert bufs[r].guards_intact()


@pytest.mark.parametrize("K,sizes,extra,in_bf16,out_bf16,order", [
    (8, [5, 2049, 7, 40000, 33], 11, True, False, RING),
    (5, [77, 30001, 1], 4, False, False, RING),
    (8, [30001, 40000, 9], 0, True, True, WIRE),
    (8, [1000000, 1500001, 3], 5, True, False, RING),   # four-slice tiles
])
def test_reduce_scatter_frags_special_values(K, sizes, extra, in_bf16, out_bf16, order):
    import torch
    total = sum(sizes)
    N = total + extra
    C = -(-N // K)
    rng = np.random.default_rng(K + N + order)
    flat = special(rng, K, total, fp32=not in_bf16)
    cuts = np.cumsum([0] + sizes)
    frags_np = [[flat[r][cuts[p]:cuts[p + 1]].copy() for p in range(len(sizes))] for r in range(K)]
    frags = [[Guarded(n, torch_dt(in_bf16), 0, frags_np[r][p]) for p, n in enumerate(sizes)]
             for r in range(K)]
    odt = np.uint16 if out_bf16 else np.float32
    outs = [Guarded(C, torch_dt(out_bf16), 0) for _ in range(K)]
    zr().zr_reduce_scatter_frags([[g.ptr() for g in row] for row in frags], sizes, N,
                                 [g.ptr() for g in outs], chunk_shift=1, average=True, order=order,
                                 in_dtype=torch_dt(in_bf16), out_dtype=torch_dt(out_bf16))
    torch.cuda.synchronize()
    bucket = oracle.flatten(frags_np, sizes, N)
    want = oracle.reduce_scatter(bucket, N, odt, shift=1, average=True, wire=(order == WIRE))
    for r in range(K):
        assert_match(outs[r].get(), want[r], f"rank {r}")
        assert outs[r].guards_intact()


@pytest.mark.parametrize("bf16", [True, False])
def test_copies_keep_every_bit(bf16):
    """All-gather and flatten of special patterns: bit for bit, NaN payloads included."""
    import torch
    K = 8
    rng = np.random.default_rng(99 if bf16 else 98)
    sizes = [8 * 2048 * 2 + 8, 5001, 1, 64]
    segs, soff, foff = [], 0, 0
    for n in sizes:
        segs.append((soff, foff, n))
        soff += -(-n // K)
        foff += n
    shard_np = special(rng, K, soff, fp32=not bf16)
    shards = [Guarded(soff, torch_dt(bf16), 0, shard_np[r]) for r in range(K)]
    fulls = [Guarded(foff, torch_dt(bf16), 0) for _ in range(K)]
    zr().zr_all_gather([g.ptr() for g in shards], [g.ptr() for g in fulls], segs, chunk_shift=0,
                       dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    dt = np.uint16 if bf16 else np.float32
    want = [np.zeros(foff, dtype=dt) for _ in range(K)]
    oracle.all_gather(shard_np, want, segs, 0)
    for r in range(K):
        assert np.array_equal(bits(fulls[r].get()), bits(want[r])), f"all-gather rank {r}"
    assert classes(want[0])["nan"] > 0

    fsizes = [3, 4096 * 3, 77, 20000]
    flat = special(rng, K, sum(fsizes), fp32=not bf16)
    cuts = np.cumsum([0] + fsizes)
    frags_np = [[flat[r][cuts[p]:cuts[p + 1]].copy() for p in range(len(fsizes))] for r in range(K)]
    frags = [[Guarded(n, torch_dt(bf16), 0, frags_np[r][p]) for p, n in enumerate(fsizes)]
             for r in range(K)]
    padded = sum(fsizes) + 13
    buckets = [Guarded(padded, torch_dt(bf16), 0) for _ in range(K)]
    zr().zr_flatten_bucket([[g.ptr() for g in row] for row in frags], fsizes,
                           [b.ptr() for b in buckets], padded, dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    wantf = oracle.flatten(frags_np, fsizes, padded)
    for r in range(K):
        assert np.array_equal(bits(buckets[r].get()), bits(wantf[r])), f"flatten rank {r}"
