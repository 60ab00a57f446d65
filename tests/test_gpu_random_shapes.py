"""Seeded random shapes through every entry point, bit-exact against the oracle.

The hand-picked parity cases pin each path; these draw the parameters at
random (per case, from a fixed seed) so the paths meet in combinations nobody
picked: K from 1 to 64, sizes from 1 element to several tiles with ragged
tails, both dtypes and every dtype pair, chunk shifts, averaging, gradient
accumulation and the bf16-wire order, base offsets shared by every rank or
different per rank (which moves calls between the vector paths, the
re-gridded paths and the aligned-pair paths for ranks in different phases),
one-shot calls and plans, with and without a workspace. K * N stays small, so
the oracle finishes each case at once.

ZR_RANDOM_SCALE multiplies the number of cases and ZR_RANDOM_SEED shifts the
seed, for a longer sweep than the default run.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import Guarded, bits

pytestmark = pytest.mark.gpu

SEED = 0x5A5200F0 + int(os.environ.get("ZR_RANDOM_SEED", "0"))
SCALE = int(os.environ.get("ZR_RANDOM_SCALE", "1"))
KS = [1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 31, 64]


def zr():
    import gradient_sync_zr_amd as m
    return m


def torch_dt(is_bf16):
    import torch
    return torch.bfloat16 if is_bf16 else torch.float32


def np_dt(is_bf16):
    return np.uint16 if is_bf16 else np.float32


def values(case, stream, n, bf16):
    """Normal values with 1% outliers (sums cancel, so the order of the fp32
    adds shows in the last bits); fp32 inputs perturb them off the bf16 grid."""
    x = synth.host_normal_bf16(SEED + case, stream, 0, n, 1.0, 0.01, 1e4)
    if bf16:
        return x
    rng = np.random.default_rng(SEED + case * 7919 + stream)
    return oracle.bf16_to_f32(x) * (1 + rng.standard_normal(n).astype(np.float32) * 1e-3)


def offsets(rng, K):
    """Element offsets of K buffers: all equal (one phase) or drawn per rank."""
    if rng.random() < 0.5:
        return [int(rng.integers(0, 4))] * K
    return [int(x) for x in rng.integers(0, 4, size=K)]


def workspace(rng, K, n):
    import torch
    if rng.random() < 0.5:
        return None
    return torch.empty(max(256, zr().zr_workspace_bytes(K, n)), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("case", range(80 * SCALE))
def test_random_reduce_scatter(case):
    import torch
    rng = np.random.default_rng(SEED + 1000 + case)
    K = int(rng.choice(KS))
    N = int(rng.integers(1, 2_000_000 // K))
    in_bf16, out_bf16 = bool(rng.random() < 0.6), bool(rng.random() < 0.4)
    shift, average = int(rng.integers(0, K)), bool(rng.random() < 0.7)
    wire = in_bf16 and rng.random() < 0.2
    steps = 2 if rng.random() < 0.3 else 1
    plan = rng.random() < 0.5
    C = -(-N // K)
    io, oo = offsets(rng, K), offsets(rng, K)
    print(f"case {case}: K={K} N={N} in_bf16={in_bf16} out_bf16={out_bf16} shift={shift} "
          f"average={average} wire={wire} steps={steps} plan={plan} in_off={io} out_off={oo}", flush=True)
    ins = [Guarded(N, torch_dt(in_bf16), io[r]) for r in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), oo[r]) for r in range(K)]
    order = zr().ZR_ORDER_RING_WIRE if wire else zr().ZR_ORDER_RING
    want = None
    for m in range(steps):
        xs = [values(case, 64 * m + r, N, in_bf16) for r in range(K)]
        for r in range(K):
            ins[r].set(xs[r])
        kw = dict(chunk_shift=shift, average=average, order=order, in_dtype=torch_dt(in_bf16),
                  out_dtype=torch_dt(out_bf16), accumulate=m > 0)
        if plan:
            p = zr().RsPlan([g.ptr() for g in ins], N, [g.ptr() for g in outs], **kw)
            p.launch()
            torch.cuda.synchronize()
            p.close()
        else:
            zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs], **kw)
        want = oracle.reduce_scatter(xs, N, np_dt(out_bf16), shift=shift, average=average, out=want,
                                     accumulate=m > 0, wire=wire)
    torch.cuda.synchronize()
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact() and ins[r].guards_intact()


@pytest.mark.parametrize("case", range(60 * SCALE))
def test_random_reduce_scatter_frags(case):
    import torch
    rng = np.random.default_rng(SEED + 2000 + case)
    K = int(rng.choice(KS))
    F = int(rng.integers(1, 41))
    cap = max(2, 1_500_000 // (K * F))
    sizes = [int(x) for x in rng.integers(0, cap, size=F)]
    total = sum(sizes)
    N = total + int(rng.integers(0, 3 * K + 1))
    if N == 0:
        N = 1
    C = -(-N // K)
    in_bf16, out_bf16 = bool(rng.random() < 0.6), bool(rng.random() < 0.4)
    shift, average = int(rng.integers(0, K)), bool(rng.random() < 0.7)
    accumulate = rng.random() < 0.25
    same = rng.random() < 0.6  # every rank's fragment p at one offset, or drawn per rank
    fo = [[int(x)] * K if same else [int(y) for y in rng.integers(0, 4, size=K)]
          for x in rng.integers(0, 4, size=F)]
    oo = offsets(rng, K)
    ws = workspace(rng, K, F)
    print(f"case {case}: K={K} F={F} sizes={sizes} N={N} in_bf16={in_bf16} out_bf16={out_bf16} "
          f"shift={shift} average={average} accumulate={accumulate} same_phase={same} "
          f"out_off={oo} ws={ws is not None}", flush=True)
    frags_np = [[values(case, 100 * r + p, n, in_bf16) for p, n in enumerate(sizes)] for r in range(K)]
    frags = [[Guarded(n, torch_dt(in_bf16), fo[p][r], frags_np[r][p]) for p, n in enumerate(sizes)]
             for r in range(K)]
    init = values(case, 9999, C, False) if accumulate else None
    outs = [Guarded(C, torch_dt(out_bf16), oo[r],
                    None if init is None else (oracle.f32_to_bf16(init) if out_bf16 else init))
            for r in range(K)]
    zr().zr_reduce_scatter_frags([[g.ptr() for g in row] for row in frags], sizes, N,
                                 [g.ptr() for g in outs], chunk_shift=shift, average=average,
                                 in_dtype=torch_dt(in_bf16), out_dtype=torch_dt(out_bf16),
                                 accumulate=accumulate, workspace=ws)
    torch.cuda.synchronize()
    prev = None
    if accumulate:
        prev = [(oracle.f32_to_bf16(init) if out_bf16 else init.copy()) for _ in range(K)]
    want = oracle.reduce_scatter(oracle.flatten(frags_np, sizes, N), N, np_dt(out_bf16), shift=shift,
                                 average=average, out=prev, accumulate=accumulate)
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()


@pytest.mark.parametrize("case", range(60 * SCALE))
def test_random_all_gather(case):
    import torch
    rng = np.random.default_rng(SEED + 3000 + case)
    K = int(rng.choice(KS))
    S = int(rng.integers(1, 12))
    bf16 = bool(rng.random() < 0.7)
    shift = int(rng.integers(0, K))
    cap = max(2, 2_000_000 // (K * S))
    segs, soff, foff = [], 0, 0
    for _ in range(S):
        n = int(rng.integers(0, cap))
        soff += int(rng.integers(0, 5))
        foff += int(rng.integers(0, 9))
        segs.append((soff, foff, n))
        soff += -(-n // K)
        foff += n
    so, fo = offsets(rng, K), offsets(rng, K)
    ws = workspace(rng, K, S)
    print(f"case {case}: K={K} bf16={bf16} shift={shift} segs={segs} shard_off={so} full_off={fo} "
          f"ws={ws is not None}", flush=True)
    shard_np = [(values(case, r, soff, True) if bf16 else values(case, r, soff, False)) for r in range(K)]
    shards = [Guarded(soff, torch_dt(bf16), so[r], shard_np[r]) for r in range(K)]
    zero = np.zeros(foff, dtype=np_dt(bf16))
    fulls = [Guarded(foff, torch_dt(bf16), fo[r], zero) for r in range(K)]
    zr().zr_all_gather([g.ptr() for g in shards], [g.ptr() for g in fulls], segs, chunk_shift=shift,
                       dtype=torch_dt(bf16), workspace=ws)
    torch.cuda.synchronize()
    want = [np.zeros(foff, dtype=np_dt(bf16)) for _ in range(K)]
    oracle.all_gather(shard_np, want, segs, shift)
    for r in range(K):
        assert np.array_equal(bits(fulls[r].get()), bits(want[r])), f"rank {r}"
        assert fulls[r].guards_intact() and shards[r].guards_intact()


@pytest.mark.parametrize("case", range(60 * SCALE))
def test_random_allreduce(case):
    import torch
    rng = np.random.default_rng(SEED + 4000 + case)
    K = int(rng.choice(KS))
    N = int(rng.integers(1, 2_000_000 // K))
    bf16, average = bool(rng.random() < 0.7), bool(rng.random() < 0.5)
    fused, inplace = bool(rng.random() < 0.7), bool(rng.random() < 0.5)
    io = offsets(rng, K)
    oo = io if inplace else offsets(rng, K)
    print(f"case {case}: K={K} N={N} bf16={bf16} average={average} fused={fused} inplace={inplace} "
          f"in_off={io} out_off={oo}", flush=True)
    xs = [values(case, r, N, bf16) for r in range(K)]
    ins = [Guarded(N, torch_dt(bf16), io[r], xs[r]) for r in range(K)]
    outs = ins if inplace else [Guarded(N, torch_dt(bf16), oo[r]) for r in range(K)]
    C = -(-N // K)
    scratch = None if fused else Guarded(K * C, torch_dt(bf16), 0)
    zr().zr_allreduce([g.ptr() for g in ins], [g.ptr() for g in outs], N, average=average, fused=fused,
                      scratch=None if scratch is None else scratch.ptr(), dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    want = oracle.allreduce(xs, N, average=average)
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()


@pytest.mark.parametrize("case", range(60 * SCALE))
def test_random_flatten(case):
    import torch
    rng = np.random.default_rng(SEED + 5000 + case)
    K = int(rng.choice(KS))
    F = int(rng.integers(1, 41))
    cap = max(2, 1_500_000 // (K * F))
    sizes = [int(x) for x in rng.integers(0, cap, size=F)]
    padded = sum(sizes) + int(rng.integers(0, 70))
    bf16 = bool(rng.random() < 0.7)
    same = rng.random() < 0.5
    fo = [[int(x)] * K if same else [int(y) for y in rng.integers(0, 4, size=K)]
          for x in rng.integers(0, 4, size=F)]
    bo = offsets(rng, K)
    ws = workspace(rng, K, F)
    print(f"case {case}: K={K} F={F} sizes={sizes} padded={padded} bf16={bf16} same_phase={same} "
          f"bucket_off={bo} ws={ws is not None}", flush=True)
    frags_np = [[values(case, 100 * r + p, n, bf16) for p, n in enumerate(sizes)] for r in range(K)]
    frags = [[Guarded(n, torch_dt(bf16), fo[p][r], frags_np[r][p]) for p, n in enumerate(sizes)]
             for r in range(K)]
    fill = np.full(padded, 0x3F80 if bf16 else 1.0, dtype=np_dt(bf16))
    buckets = [Guarded(padded, torch_dt(bf16), bo[r], fill) for r in range(K)]
    zr().zr_flatten_bucket([[g.ptr() for g in row] for row in frags], sizes, [g.ptr() for g in buckets],
                           padded, dtype=torch_dt(bf16), workspace=ws)
    torch.cuda.synchronize()
    want = oracle.flatten(frags_np, sizes, padded)
    for r in range(K):
        assert np.array_equal(bits(buckets[r].get()), bits(want[r])), f"rank {r}"
        assert buckets[r].guards_intact()
