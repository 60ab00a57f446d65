"""GPU parity of every entry point against the CPU oracle, at sizes the oracle
finishes in seconds: several 2048-element tiles plus ragged tails, misaligned
bases (tile grids shifted onto them), every dtype pair, chunk shifts, averaging,
K from 1 to 64, and the degenerate cases (N = 0, N < K, K = 1).

Ring order must match the oracle bit for bit; the free order must lie within
1e-5 of the sum of magnitudes (/K when averaging) of the exact sum, plus one
bf16 ulp for bf16 outputs. Every buffer is guarded by a sentinel band.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Guarded, bf16_ulp, bits

pytestmark = pytest.mark.gpu

SEED = 0x5A5200A0


def zr():
    import gradient_sync_zr_amd as m
    return m


def workspace(use, K, n):
    """A device workspace for a call with n fragments or segments (None when
    `use` is false): the size zr_workspace_bytes asks for, at least 256 bytes."""
    import torch
    if not use:
        return None
    return torch.empty(max(256, zr().zr_workspace_bytes(K, n)), dtype=torch.uint8, device="cuda")


def torch_dt(is_bf16):
    import torch
    return torch.bfloat16 if is_bf16 else torch.float32


def make_inputs(K, N, bf16, case):
    """Normal values with 1% of large outliers: sums cancel, so the order of
    fp32 additions shows in the last bits."""
    xs = [synth.host_normal_bf16(SEED + case, r, 0, N, 1.0, 0.01, 1e4) for r in range(K)]
    if bf16:
        return xs
    rng = np.random.default_rng(case)
    return [oracle.bf16_to_f32(x) * (1 + rng.standard_normal(N).astype(np.float32) * 1e-3)
            for x in xs]


RS_CASES = [
    # K, N, in_bf16, out_bf16, shift, average, offset
    (1, 1000, True, False, 0, True, 0),
    (2, 2, True, False, 1, True, 0),
    (3, 2, True, False, 1, False, 0),           # N < K: last chunk(s) all padding
    (4, 16, False, False, 1, False, 0),
    (8, 8 * 2048 * 3, True, False, 1, True, 0),  # exact tiles
    (8, 8 * 2048 * 3 + 8 * 13, True, False, 1, True, 0),  # C % 8 != 0 ... ragged
    (8, 8 * 2048 * 2 + 61, True, False, 1, True, 0),      # ragged tail, padding
    (8, 100003, True, True, 1, True, 0),
    (8, 100003, False, False, 0, True, 0),
    (8, 100003, False, True, 3, False, 0),
    (8, 65536, True, False, 1, True, 1),         # bases off the quad grid: the discrete path's tiles
    (8, 65536 + 5, False, False, 1, True, 3),
    (5, 77777, True, False, 2, True, 0),         # non power of two: IEEE divide
    (3, 50001, False, True, 1, True, 0),
    (7, 7 * 4096, True, False, 6, True, 0),
    (16, 16 * 2048 + 3, True, False, 1, True, 0),
    (16, 160000, True, True, 15, False, 0),
    (64, 64 * 2048 + 17, True, False, 1, True, 0),
    (64, 300007, True, True, 1, False, 0),
    (64, 200000, False, False, 0, True, 1),
    (33, 33 * 3000 + 1, True, False, 1, True, 0),
    # large enough for full four-slice tiles (smaller launches use one slice)
    (8, 8 * 300000 + 13, True, False, 1, True, 0),
    (16, 16 * 150000 + 5, False, True, 1, True, 0),
    (64, 64 * 40000 + 7, True, False, 1, False, 0),
    # K > 8 with chunk starts off the quad grid (C mod 4 = 2, 3, 2): these go
    # out as a discrete reduce-scatter over one fragment per rank
    (32, 32 * 50002, True, False, 1, True, 0),
    (32, 32 * 50003 - 5, True, True, 3, True, 0),
    (17, 17 * 20001 + 2, True, False, 1, True, 0),
]


@pytest.mark.parametrize("entry", ["call", "plan"])
@pytest.mark.parametrize("K,N,in_bf16,out_bf16,shift,average,offset", RS_CASES)
def test_reduce_scatter_ring_bit_exact(K, N, in_bf16, out_bf16, shift, average, offset, entry):
    # the one-shot call, and a plan built once and launched twice
    import torch
    case = K * 1000003 + N
    xs = make_inputs(K, N, in_bf16, case)
    C = -(-N // K)
    ins = [Guarded(N, torch_dt(in_bf16), offset, xs[r]) for r in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), offset) for _ in range(K)]
    kw = dict(chunk_shift=shift, average=average, in_dtype=torch_dt(in_bf16),
              out_dtype=torch_dt(out_bf16))
    if entry == "call":
        zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs], **kw)
    else:
        plan = zr().RsPlan([g.ptr() for g in ins], N, [g.ptr() for g in outs], **kw)
        plan.launch()
        torch.cuda.synchronize()
        for g in outs:
            g.t.view(torch.int16 if out_bf16 else torch.int32).fill_(-1)
        plan.launch()
        plan.close()
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(xs, N, np.uint16 if out_bf16 else np.float32, shift=shift,
                                 average=average)
    for r in range(K):
        got = outs[r].get()
        assert np.array_equal(bits(got), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact() and ins[r].guards_intact()


ACC_CASES = [
    # K, N, in_bf16, out_bf16, shift, average, offset
    (8, 8 * 4096 * 3 + 8 * 40, True, False, 1, True, 0),
    (8, 100003, True, True, 1, True, 0),
    (5, 77777, False, False, 2, True, 0),
    (8, 65536 + 5, True, False, 0, False, 1),     # bases off the quad grid
    (64, 64 * 4096 + 3, True, False, 1, True, 0),
    (3, 2, True, False, 1, True, 0),
    (8, 8 * 300000 + 13, True, False, 1, True, 0),   # four-slice tiles
]


@pytest.mark.parametrize("K,N,in_bf16,out_bf16,shift,average,offset", ACC_CASES)
def test_reduce_scatter_accumulate_bit_exact(K, N, in_bf16, out_bf16, shift, average, offset):
    # gradient accumulation: micro-step 0 overwrites, micro-steps 1.. add in place
    import torch
    C = -(-N // K)
    steps = [make_inputs(K, N, in_bf16, 777 + K + N + m) for m in range(3)]
    ins = [Guarded(N, torch_dt(in_bf16), offset) for _ in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), offset) for _ in range(K)]
    want = None
    for m, xs in enumerate(steps):
        for r in range(K):
            ins[r].set(xs[r])
        zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs],
                                   chunk_shift=shift, average=average, accumulate=m > 0,
                                   in_dtype=torch_dt(in_bf16), out_dtype=torch_dt(out_bf16))
        want = oracle.reduce_scatter(xs, N, np.uint16 if out_bf16 else np.float32, shift=shift,
                                     average=average, out=want, accumulate=m > 0)
    torch.cuda.synchronize()
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()


WIRE_CASES = [
    # K, N, out_bf16, shift, average, offset
    (8, 8 * 4096 * 3 + 8 * 40, False, 1, True, 0),
    (8, 100003, True, 1, False, 0),
    (8, 65536 + 5, False, 0, True, 1),          # bases off the quad grid
    (5, 77777, False, 2, True, 0),
    (64, 64 * 4096 + 3, True, 1, False, 0),
    # full tiles of the generic wire kernels (four ranks per batch; bf16
    # output on four-slice tiles)
    (3, 3 * 400001, True, 1, True, 0),
    (16, 16 * 150000 + 5, True, 1, True, 0),
    (16, 16 * 150000 + 5, False, 2, False, 0),
]


@pytest.mark.parametrize("K,N,out_bf16,shift,average,offset", WIRE_CASES)
def test_reduce_scatter_bf16_wire_bit_exact(K, N, out_bf16, shift, average, offset):
    import torch
    xs = make_inputs(K, N, True, 4242 + K + N)
    C = -(-N // K)
    ins = [Guarded(N, torch.bfloat16, offset, xs[r]) for r in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), offset) for _ in range(K)]
    zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs],
                               chunk_shift=shift, average=average, order=zr().ZR_ORDER_RING_WIRE,
                               in_dtype=torch.bfloat16, out_dtype=torch_dt(out_bf16))
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(xs, N, np.uint16 if out_bf16 else np.float32, shift=shift,
                                 average=average, wire=True)
    ring = oracle.reduce_scatter(xs, N, np.uint16 if out_bf16 else np.float32, shift=shift,
                                 average=average)
    differs = False
    for r in range(K):
        got = outs[r].get()
        assert np.array_equal(bits(got), bits(want[r])), f"rank {r}"
        differs |= not np.array_equal(bits(got), bits(ring[r]))
        assert outs[r].guards_intact()
    assert differs  # per-hop rounding shows on these inputs


@pytest.mark.parametrize("K,N,fused,average", [(8, 8 * 4096 * 2 + 77, True, False),
                                               (8, 8 * 4096 * 2 + 77, False, True),
                                               (64, 64 * 4096 + 9, True, False),
                                               (3, 30001, True, True)])
def test_allreduce_bf16_wire_bit_exact(K, N, fused, average):
    import torch
    xs = make_inputs(K, N, True, 5151 + K + N)
    ins = [Guarded(N, torch.bfloat16, 0, xs[r]) for r in range(K)]
    C = -(-N // K)
    scratch = None if fused else Guarded(K * C, torch.bfloat16, 0)
    zr().zr_allreduce([g.ptr() for g in ins], [g.ptr() for g in ins], N, average=average,
                      order=zr().ZR_ORDER_RING_WIRE, fused=fused,
                      scratch=None if scratch is None else scratch.ptr(), dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.allreduce(xs, N, average=average, wire=True)
    for r in range(K):
        assert np.array_equal(ins[r].get(), want[r]), f"rank {r}"


@pytest.mark.parametrize("K,N,in_bf16,out_bf16,average", [
    (8, 100003, True, False, True), (64, 70001, True, True, False), (5, 30000, False, False, True),
    (16, 16 * 2048 * 2, True, False, True),
    # full tiles: bf16 -> bf16 takes four-slice tiles in the free order
    (8, 8 * 300000 + 13, True, True, True), (2, 2 * 500000 + 1, True, True, False),
    (3, 3 * 200001, True, False, True), (64, 64 * 20000 + 5, False, True, True)])
def test_reduce_scatter_free_order_within_tolerance(K, N, in_bf16, out_bf16, average):
    import torch
    xs = make_inputs(K, N, in_bf16, 77 + K)
    C = -(-N // K)
    ins = [Guarded(N, torch_dt(in_bf16), 0, xs[r]) for r in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), 0) for _ in range(K)]
    zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs], chunk_shift=1,
                               average=average, order=zr().ZR_ORDER_FREE,
                               in_dtype=torch_dt(in_bf16), out_dtype=torch_dt(out_bf16))
    torch.cuda.synchronize()
    xf = np.stack([oracle.bf16_to_f32(x) if in_bf16 else x for x in xs])
    xp = np.zeros((K, K * C), dtype=np.float32)
    xp[:, :N] = xf
    exact, absum = oracle.exact_sum_points(xp)
    scale = 1.0 / K if average else 1.0
    ring = oracle.reduce_scatter(xs, N, np.float32, shift=1, average=average)
    differs = False
    for q in range(K):
        j = (q + 1) % K
        got = outs[q].get()
        gotf = oracle.bf16_to_f32(got) if out_bf16 else got
        ex = exact[j * C:(j + 1) * C] * scale
        tol = 1e-5 * absum[j * C:(j + 1) * C] * scale
        if out_bf16:
            tol = tol + bf16_ulp(ex)
        assert np.all(np.abs(gotf.astype(np.float64) - ex) <= tol), f"rank {q}"
        differs |= not np.array_equal(bits(gotf.astype(np.float32)), bits(ring[q]))
        assert outs[q].guards_intact()
    if K >= 16 and not out_bf16:
        assert differs  # the free order is a different order


AR_CASES = [
    # K, N, bf16, average, fused, inplace, offset
    (4, 16, False, False, True, False, 0),
    (4, 16, False, False, False, False, 0),
    (8, 8 * 2048 * 4, True, False, True, True, 0),
    (8, 8 * 2048 * 4 + 77, True, True, True, False, 0),
    (8, 8 * 2048 * 4 + 77, True, True, False, True, 0),
    (8, 123457, False, False, True, True, 0),
    # bases off the quad grid, all in one phase: the tile grid starts `lead` in
    (8, 123457, True, False, True, True, 1),
    (8, 8 * 2048 * 4 + 77, True, True, True, False, 2),
    (8, 8 * 2048 * 4 + 77, True, True, True, True, 3),
    (8, 99999, False, False, True, False, 1),
    (8, 99999, False, True, True, True, 2),
    (8, 99999, False, False, True, True, 3),
    (64, 64 * 2048 + 9, True, False, True, True, 1),
    (4, 2, True, False, True, True, 1),        # N < lead: no tiles, one block
    (4, 5, False, False, True, False, 3),
    (3, 30001, True, True, True, False, 0),
    (64, 64 * 2048 + 9, True, False, True, True, 0),
    (64, 200003, True, False, False, True, 0),
    (64, 1000, True, False, True, False, 0),   # C < tile: every tile straddles chunks
    (1, 5000, True, True, True, True, 0),
    (2, 1, False, False, True, True, 0),
    (17, 17 * 2048 + 1, False, True, True, False, 0),
]


@pytest.mark.parametrize("K,N,bf16,average,fused,inplace,offset", AR_CASES)
def test_allreduce_bit_exact(K, N, bf16, average, fused, inplace, offset):
    import torch
    xs = make_inputs(K, N, bf16, 5000 + K * 7 + N)
    ins = [Guarded(N, torch_dt(bf16), offset, xs[r]) for r in range(K)]
    outs = ins if inplace else [Guarded(N, torch_dt(bf16), offset) for _ in range(K)]
    C = -(-N // K)
    scratch = None if fused else Guarded(K * C, torch_dt(bf16), 0)
    zr().zr_allreduce([g.ptr() for g in ins], [g.ptr() for g in outs], N, average=average,
                      fused=fused, scratch=None if scratch is None else scratch.ptr(),
                      dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    want = oracle.allreduce(xs, N, average=average)
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()
    if scratch is not None:
        assert scratch.guards_intact()


@pytest.mark.parametrize("bf16", [True, False])
def test_allreduce_ranks_in_different_phases(bf16):
    # bases in different phases within a quad: no common tile grid, so every
    # rank's quad is read as an aligned pair and every output realigned in LDS
    import torch
    K, N = 8, 50003
    xs = make_inputs(K, N, bf16, 777)
    ins = [Guarded(N, torch_dt(bf16), r % 4, xs[r]) for r in range(K)]
    outs = [Guarded(N, torch_dt(bf16), (r + 1) % 4) for r in range(K)]
    zr().zr_allreduce([g.ptr() for g in ins], [g.ptr() for g in outs], N, average=True, fused=True,
                      dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    want = oracle.allreduce(xs, N, average=True)
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()


@pytest.mark.parametrize("K,N,bf16", [(8, 99991, True), (64, 64 * 2048 * 2 + 5, True),
                                      (5, 44444, False)])
def test_allreduce_fused_equals_rs_then_ag(K, N, bf16):
    # all-reduce = reduce-scatter then all-gather (lecture 14, 2.2), on the GPU
    import torch
    xs = make_inputs(K, N, bf16, 9000 + K)
    ins = [Guarded(N, torch_dt(bf16), 0, xs[r]) for r in range(K)]
    a = [Guarded(N, torch_dt(bf16), 0) for _ in range(K)]
    b = [Guarded(N, torch_dt(bf16), 0) for _ in range(K)]
    C = -(-N // K)
    sh = [Guarded(C, torch_dt(bf16), 0) for _ in range(K)]
    m = zr()
    m.zr_allreduce([g.ptr() for g in ins], [g.ptr() for g in a], N, fused=True,
                   dtype=torch_dt(bf16))
    m.zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in sh], chunk_shift=1,
                            average=False, in_dtype=torch_dt(bf16), out_dtype=torch_dt(bf16))
    m.zr_all_gather([g.ptr() for g in sh], [g.ptr() for g in b], [(0, 0, N)], chunk_shift=1,
                    dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    ref = a[0].get()
    for r in range(K):
        assert np.array_equal(bits(a[r].get()), bits(b[r].get()))
        assert np.array_equal(bits(a[r].get()), bits(ref))   # identical on every rank


@pytest.mark.parametrize("K,N", [(64, 64 * 2048 + 999), (8, 8 * 8192 * 20 + 3), (3, 3 * 8192 * 9 + 1)])
def test_allreduce_free_order_tolerance_and_identical_ranks(K, N):
    import torch
    xs = make_inputs(K, N, True, 31337 + K)
    ins = [Guarded(N, torch.bfloat16, 0, xs[r]) for r in range(K)]
    zr().zr_allreduce([g.ptr() for g in ins], [g.ptr() for g in ins], N,
                      order=zr().ZR_ORDER_FREE, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xf = np.stack([oracle.bf16_to_f32(x) for x in xs])
    exact, absum = oracle.exact_sum_points(xf)
    ref = ins[0].get()
    got = oracle.bf16_to_f32(ref).astype(np.float64)
    assert np.all(np.abs(got - exact) <= 1e-5 * absum + bf16_ulp(exact))
    for r in range(1, K):
        assert np.array_equal(ins[r].get(), ref)


AG_CASES = [
    # K, sizes, shift, bf16, offset, full gap
    (8, [8 * 2048 * 2, 8 * 2048 * 3 + 8, 5000, 1, 7], 0, True, 0, 0),
    (8, [100003, 64, 3], 1, True, 0, 3),
    (8, [65536] * 40, 0, True, 0, 0),          # more than one launch of segments
    (4, [1000 + 37 * i for i in range(150)], 1, True, 0, 1),  # 150 segments: one staged launch
    (3, [10, 30001, 2], 2, False, 1, 1),
    (64, [64 * 2048 + 5, 640, 63], 0, True, 0, 0),
    (1, [12345], 0, True, 0, 0),
    (5, [0, 4, 0, 99999], 3, True, 1, 2),
    # fp32 over several 4096-element tiles per chunk, odd sizes (16-byte units of 4 elements)
    (8, [8 * 4096 * 3 + 5, 77, 8 * 1024 + 1], 1, False, 0, 1),
    (16, [16 * 4096 * 2 + 3, 16 * 4096], 5, False, 3, 2),
]


@pytest.mark.parametrize("ws", [False, True], ids=["args", "workspace"])
@pytest.mark.parametrize("K,sizes,shift,bf16,offset,gap", AG_CASES)
def test_all_gather_bit_exact(K, sizes, shift, bf16, offset, gap, ws):
    import torch
    rng = np.random.default_rng(sum(sizes) + K)
    segs, soff, foff = [], 0, 0
    for n in sizes:
        segs.append((soff, foff, n))
        soff += -(-n // K) + gap
        foff += n + gap
    dt = np.uint16 if bf16 else np.float32
    shard_np = [(rng.integers(0, 65535, size=soff).astype(np.uint16) if bf16 else
                 rng.standard_normal(soff).astype(np.float32)) for _ in range(K)]
    shards = [Guarded(soff, torch_dt(bf16), offset, shard_np[r]) for r in range(K)]
    fill = np.zeros(foff, dtype=dt)
    fulls = [Guarded(foff, torch_dt(bf16), offset, fill) for _ in range(K)]
    zr().zr_all_gather([g.ptr() for g in shards], [g.ptr() for g in fulls], segs,
                       chunk_shift=shift, dtype=torch_dt(bf16), workspace=workspace(ws, K, len(segs)))
    torch.cuda.synchronize()
    want = [np.zeros(foff, dtype=dt) for _ in range(K)]
    oracle.all_gather(shard_np, want, segs, shift)
    for r in range(K):
        assert np.array_equal(bits(fulls[r].get()), bits(want[r])), f"rank {r}"
        assert fulls[r].guards_intact() and shards[r].guards_intact()


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("ws", [False, True], ids=["args", "workspace"])
def test_all_gather_every_phase_pair(bf16, ws):
    # one segment per (shard phase, full phase) within 16 bytes, each large
    # enough that its chunks span two tiles with ragged ends, so whole groups
    # are loaded from every source phase (one aligned block, or two or three
    # joined in registers) and stored to every destination grid
    import torch
    K = 8
    per = 8 if bf16 else 4  # elements per 16 bytes
    n = 8 * (8192 if bf16 else 4096) + 13
    segs, soff, foff = [], 0, 0
    for ps in range(per):
        for pf in range(per):
            soff += (ps - soff) % per
            foff += (pf - foff) % per
            segs.append((soff, foff, n))
            soff += -(-n // K)
            foff += n
    dt = np.uint16 if bf16 else np.float32
    rng = np.random.default_rng(4242 + per)
    shard_np = [(rng.integers(0, 65535, size=soff).astype(np.uint16) if bf16 else
                 rng.standard_normal(soff).astype(np.float32)) for _ in range(K)]
    shards = [Guarded(soff, torch_dt(bf16), 0, shard_np[r]) for r in range(K)]
    fulls = [Guarded(foff, torch_dt(bf16), 0, np.zeros(foff, dtype=dt)) for _ in range(K)]
    zr().zr_all_gather([g.ptr() for g in shards], [g.ptr() for g in fulls], segs, chunk_shift=1,
                       dtype=torch_dt(bf16), workspace=workspace(ws, K, len(segs)))
    torch.cuda.synchronize()
    want = [np.zeros(foff, dtype=dt) for _ in range(K)]
    oracle.all_gather(shard_np, want, segs, 1)
    for r in range(K):
        assert np.array_equal(bits(fulls[r].get()), bits(want[r])), f"rank {r}"
        assert fulls[r].guards_intact() and shards[r].guards_intact()


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("full_offsets", ["shared", "mixed"])
def test_all_gather_views_off_the_grid(bf16, full_offsets):
    # every shard at its own phase (a chunk reads one shard, so any phase is
    # shifted into place); the full buffers at one shared odd phase (whole
    # groups on their common grid) or at mixed phases (each tile's source
    # staged in LDS and shifted per destination)
    import torch
    K = 8
    sizes = [8 * 8192 * 2 + 13, 999, 8 * 4096 + 7]
    segs, soff, foff = [], 0, 0
    for n in sizes:
        segs.append((soff, foff, n))
        soff += -(-n // K) + 1
        foff += n + 3
    dt = np.uint16 if bf16 else np.float32
    rng = np.random.default_rng(99 + K)
    shard_np = [(rng.integers(0, 65535, size=soff).astype(np.uint16) if bf16 else
                 rng.standard_normal(soff).astype(np.float32)) for _ in range(K)]
    shards = [Guarded(soff, torch_dt(bf16), r % 8, shard_np[r]) for r in range(K)]
    fo = (lambda r: 3) if full_offsets == "shared" else (lambda r: (r * 3) % 8)
    fulls = [Guarded(foff, torch_dt(bf16), fo(r), np.zeros(foff, dtype=dt)) for r in range(K)]
    zr().zr_all_gather([g.ptr() for g in shards], [g.ptr() for g in fulls], segs, chunk_shift=1,
                       dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    want = [np.zeros(foff, dtype=dt) for _ in range(K)]
    oracle.all_gather(shard_np, want, segs, 1)
    for r in range(K):
        assert np.array_equal(bits(fulls[r].get()), bits(want[r])), f"rank {r}"
        assert fulls[r].guards_intact() and shards[r].guards_intact()


@pytest.mark.parametrize("K,sizes,bf16,offset,extra", [
    (8, None, True, 0, None),                      # the 64 log-uniform fragments
    (3, [5, 0, 1, 2049, 7, 4096, 33], True, 0, 11),
    (4, [8, 16, 24, 4096 * 3], False, 0, 4),       # aligned: 16-byte copies
    (2, [1000, 3, 5], True, 1, 0),
    (64, [100, 1], True, 0, 27),
    # a launch carries 32 fragments' rank pointers (4 at K = 64) and the
    # padding in a spare slot after them
    (8, [97 * (i + 1) for i in range(32)], True, 0, 20000),
    (8, [50 + 13 * i for i in range(33)], False, 1, 9),
    (64, [3000 + i for i in range(9)], True, 0, 100),
    (16, [], True, 0, 777),                        # padding only
    # launches large enough for 16 KiB tiles
    (8, [600000, 5, 700001], True, 0, 3),
    (4, [300001, 7, 500000], False, 1, 0),
    (64, [1 + 97 * i for i in range(40)], True, 0, 5),  # ten argument launches, or one staged
])
@pytest.mark.parametrize("ws", [False, True], ids=["args", "workspace"])
def test_flatten_bit_exact(K, sizes, bf16, offset, extra, ws):
    import torch
    from synth import workloads as W
    if sizes is None:
        sizes = W.flatten8_numels()
    total = sum(sizes)
    padded = -(-total // K) * K if extra is None else total + extra
    frags_np = []
    for r in range(K):
        row = []
        for p, n in enumerate(sizes):
            h = synth.host_normal_bf16(SEED, W.flatten8_frag_stream(r, p), 0, n, 1e-3)
            row.append(h if bf16 else oracle.bf16_to_f32(h))
        frags_np.append(row)
    frags = [[Guarded(n, torch_dt(bf16), offset, frags_np[r][p]) for p, n in enumerate(sizes)]
             for r in range(K)]
    buckets = [Guarded(padded, torch_dt(bf16), offset,
                       np.full(padded, 0x3F80 if bf16 else 1.0,
                               dtype=np.uint16 if bf16 else np.float32)) for _ in range(K)]
    zr().zr_flatten_bucket([[g.ptr() for g in row] for row in frags], sizes,
                           [b.ptr() for b in buckets], padded, dtype=torch_dt(bf16),
                           workspace=workspace(ws, K, len(sizes)))
    torch.cuda.synchronize()
    want = oracle.flatten(frags_np, sizes, padded)
    for r in range(K):
        assert np.array_equal(bits(buckets[r].get()), bits(want[r])), f"rank {r}"
        assert buckets[r].guards_intact()


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("ws", [False, True], ids=["args", "workspace"])
def test_flatten_every_phase_pair(bf16, ws):
    # every (source, destination) phase within 16 bytes: fragments are views
    # at element offsets 0..per-1 into one buffer per rank, and their bucket
    # offsets (prefix sums of their sizes) fall in every phase; each pair is
    # copied by whole realigned units between partial first and last units
    import torch
    K = 4
    per = 8 if bf16 else 4
    F = per * per
    rng = np.random.default_rng(4242 + bf16)
    # fragment p: source phase p % per, bucket phase p // per (sizes chosen so
    # the prefix sums land there, gaps in the buffers so the views do)
    sizes = []
    for p_ in range(F):
        delta = ((p_ + 1) // per - p_ // per) % per
        sizes.append(per * int(rng.integers(0, 300)) + delta or per)
    dt = np.uint16 if bf16 else np.float32
    frags_np, fp, bufs, pairs = [], [], [], set()
    for r in range(K):
        row = [synth.host_normal_bf16(SEED + 17, r * 4096 + p_, 0, n, 1.0) for p_, n in enumerate(sizes)]
        row = row if bf16 else [oracle.bf16_to_f32(h) for h in row]
        frags_np.append(row)
        offs, o = [], 0
        for p_, n in enumerate(sizes):
            o += (p_ - o) % per
            offs.append(o)
            o += n
        host = np.zeros(o, dtype=dt)
        for p_, n in enumerate(sizes):
            host[offs[p_]:offs[p_] + n] = row[p_]
        g = Guarded(o, torch_dt(bf16), 0, host)
        bufs.append(g)
        es = 2 if bf16 else 4
        fp.append([g.ptr() + es * offs[p_] for p_ in range(F)])
        boff = 0
        for p_, n in enumerate(sizes):
            pairs.add(((g.ptr() + es * offs[p_]) % 16 // es, (boff * es) % 16 // es))
            boff += n
    assert len(pairs) == per * per, sorted(pairs)  # the bucket and the buffers start 256-byte aligned
    padded = sum(sizes) + 7
    buckets = [Guarded(padded, torch_dt(bf16), 0, np.full(padded, 0x3F80 if bf16 else 1.0, dtype=dt))
               for _ in range(K)]
    zr().zr_flatten_bucket(fp, sizes, [b.ptr() for b in buckets], padded, dtype=torch_dt(bf16),
                           workspace=workspace(ws, K, F))
    torch.cuda.synchronize()
    want = oracle.flatten(frags_np, sizes, padded)
    for r in range(K):
        assert np.array_equal(bits(buckets[r].get()), bits(want[r])), f"rank {r}"
        assert buckets[r].guards_intact() and bufs[r].guards_intact()


FRAG_CASES = [
    # K, sizes (None = the 64 log-uniform fragments), extra padding, in_bf16, out_bf16,
    # shift, average, order, offset, accumulate
    (8, None, None, True, False, 1, True, 0, 0, False),
    (8, [5, 0, 1, 2049, 7, 4096 * 3, 33, 64], 11, True, False, 1, True, 0, 0, False),
    (8, [4096, 8192, 16, 24], 0, True, True, 0, False, 0, 0, False),
    (8, [1000, 3, 5, 100000], 3, True, False, 1, True, 0, 1, False),   # misaligned fragments
    (5, [77, 7777, 1], 4, False, False, 2, True, 0, 0, False),
    (64, [100, 1, 4096 * 5 + 3, 64 * 7], 64 * 3, True, False, 1, True, 0, 0, False),
    (8, [30001, 40000], 7, True, False, 1, True, 2, 0, False),        # bf16 wire order
    (16, [30001, 40000], 0, True, False, 1, True, 1, 0, False),       # free order
    (8, [30001, 40000, 9], 0, True, False, 1, True, 0, 0, True),      # accumulate
    (3, [], 10, True, False, 1, True, 0, 0, False),                   # padding only
    (64, [300000, 5], 59, True, False, 1, True, 0, 0, False),         # K = 64 vector tiles
    (8, [30001, 40000, 9], 5, True, True, 1, True, 0, -1, False),     # ranks in different quad phases
    (8, [6, 30000, 40000], 2, True, True, 1, True, 0, 0, False),      # bf16 partition side unaligned
    (8, [6, 30000, 40000], 2, False, False, 1, True, 0, 0, True),     # fp32, unaligned, accumulate
    (8, [6, 30000, 40000], 2, True, False, 0, True, 2, -1, False),    # wire order, mixed phases
    (8, [1000000, 1500001, 3], 5, True, False, 1, True, 0, 0, False), # four-slice tiles
    (8, [1000000, 1500001, 3], 5, True, False, 1, True, 0, 0, True),  # four-slice, accumulate
    # the padding entry takes the slot after the last fragment of a launch
    (8, [97 * (i + 1) for i in range(32)], 20000, True, False, 1, True, 0, 0, False),  # over 3 chunks
    (8, [50 + 13 * i for i in range(33)], 9, True, False, 1, True, 0, 0, True),  # 32 + (1 + padding)
    (64, [32000] * 6, 64 * 40, True, False, 1, True, 0, 0, False),     # 4 fragments per launch
    # many fragments at K = 64: 16 argument launches, or one over a staged table
    (64, [1 + 613 * i for i in range(64)], 64 * 7, True, False, 1, True, 0, 0, False),
    (64, [1 + 613 * i for i in range(64)], 64 * 7, True, True, 1, True, 2, -1, True),
]


@pytest.mark.parametrize("ws", [False, True], ids=["args", "workspace"])
@pytest.mark.parametrize("K,sizes,extra,in_bf16,out_bf16,shift,average,order,offset,acc",
                         FRAG_CASES)
def test_reduce_scatter_frags_bit_exact(K, sizes, extra, in_bf16, out_bf16, shift, average,
                                        order, offset, acc, ws):
    # the discrete path equals flatten-into-a-bucket then reduce-scatter;
    # offset -1: rank r's fragments at element offset r % 4 (the ranks' buffers
    # in different quad phases), every partition at offset 1
    import torch
    from synth import workloads as W
    if sizes is None:
        sizes = W.flatten8_numels()
    total = sum(sizes)
    N = -(-total // K) * K if extra is None else total + extra
    C = -(-N // K)
    frags_np = []
    for r in range(K):
        row = []
        for p, n in enumerate(sizes):
            h = synth.host_normal_bf16(SEED + 77, r * 4096 + p, 0, n, 1.0, 0.01, 1e4)
            row.append(h if in_bf16 else oracle.bf16_to_f32(h))
        frags_np.append(row)
    f_off = (lambda r: r % 4) if offset == -1 else (lambda r: offset)
    o_off = 1 if offset == -1 else offset
    frags = [[Guarded(n, torch_dt(in_bf16), f_off(r), frags_np[r][p]) for p, n in enumerate(sizes)]
             for r in range(K)]
    odt = np.uint16 if out_bf16 else np.float32
    rng = np.random.default_rng(K + N)
    init = [oracle.f32_to_bf16(rng.standard_normal(C).astype(np.float32)) if out_bf16 else
            rng.standard_normal(C).astype(np.float32) for _ in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), o_off, init[r]) for r in range(K)]
    zr().zr_reduce_scatter_frags([[g.ptr() for g in row] for row in frags], sizes, N,
                                 [g.ptr() for g in outs], chunk_shift=shift, average=average,
                                 order=order, accumulate=acc, in_dtype=torch_dt(in_bf16),
                                 out_dtype=torch_dt(out_bf16), workspace=workspace(ws, K, len(sizes)))
    torch.cuda.synchronize()
    bucket = oracle.flatten(frags_np, sizes, N) if sizes else \
        [np.zeros(N, dtype=np.uint16 if in_bf16 else np.float32) for _ in range(K)]
    if order == 1:
        # free order: the discrete call, and the contiguous free-order call on
        # the bucket the flatten would build, are each within the free-order
        # bound of the oracle's exact (fp64) sum
        assert not acc
        bt = [Guarded(N, torch_dt(in_bf16), 0, bucket[r]) for r in range(K)]
        ref = [Guarded(C, torch_dt(out_bf16), 0) for _ in range(K)]
        zr().zr_reduce_scatter_avg([g.ptr() for g in bt], N, [g.ptr() for g in ref],
                                   chunk_shift=shift, average=average, order=1,
                                   in_dtype=torch_dt(in_bf16), out_dtype=torch_dt(out_bf16))
        torch.cuda.synchronize()
        xf = np.stack([oracle.bf16_to_f32(x) if in_bf16 else x for x in bucket])
        xp = np.zeros((K, K * C), dtype=np.float32)
        xp[:, :N] = xf
        exact, absum = oracle.exact_sum_points(xp)
        scale = 1.0 / K if average else 1.0
        for q in range(K):
            j = (q + shift) % K
            ex = exact[j * C:(j + 1) * C] * scale
            bound = 1e-5 * absum[j * C:(j + 1) * C] * scale + (bf16_ulp(ex) if out_bf16 else 0)
            for name, res in (("discrete", outs[q]), ("contiguous", ref[q])):
                got = res.get()
                gotf = (oracle.bf16_to_f32(got) if out_bf16 else got).astype(np.float64)
                assert np.all(np.abs(gotf - ex) <= bound), f"{name} free order, rank {q}"
        return
    want = [x.copy() for x in init]
    oracle.reduce_scatter(bucket, N, odt, shift=shift, average=average, out=want,
                          accumulate=acc, wire=(order == 2))
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()
    for row in frags:
        for g in row:
            assert g.guards_intact()


@pytest.mark.parametrize("case", [FRAG_CASES[i] for i in (0, 1, 3, 5, 6, 7, 8, 11, 13, 17, 18, 19)])
def test_rsf_plan_launches_equal_the_call(case):
    # a plan built once, launched twice (the fragments rewritten in place in
    # between), against the one-shot call with the same arguments each time
    import torch
    import gradient_sync_zr_amd as zrm
    from synth import workloads as W
    K, sizes, extra, in_bf16, out_bf16, shift, average, order, offset, acc = case
    if sizes is None:
        sizes = W.flatten8_numels()
    total = sum(sizes)
    N = -(-total // K) * K if extra is None else total + extra
    C = -(-N // K)
    f_off = (lambda r: r % 4) if offset == -1 else (lambda r: offset)
    o_off = 1 if offset == -1 else offset
    frags = [[Guarded(n, torch_dt(in_bf16), f_off(r)) for n in sizes] for r in range(K)]

    def fill(tag):
        for r in range(K):
            for p, n in enumerate(sizes):
                h = synth.host_normal_bf16(SEED + 300 + tag, r * 4096 + p, 0, n, 1.0, 0.01, 1e4)
                frags[r][p].set(h if in_bf16 else oracle.bf16_to_f32(h))
    rng = np.random.default_rng(K + N + 1)
    init = [rng.standard_normal(C).astype(np.float32) for _ in range(K)]
    if out_bf16:
        init = [oracle.f32_to_bf16(x) for x in init]
    by_call = [Guarded(C, torch_dt(out_bf16), o_off, init[r]) for r in range(K)]
    by_plan = [Guarded(C, torch_dt(out_bf16), o_off, init[r]) for r in range(K)]
    fp = [[g.ptr() for g in row] for row in frags]
    kw = dict(chunk_shift=shift, average=average, order=order, accumulate=acc,
              in_dtype=torch_dt(in_bf16), out_dtype=torch_dt(out_bf16))
    plan = zrm.RsfPlan(fp, sizes, N, [g.ptr() for g in by_plan], **kw)
    for tag in (0, 1):
        fill(tag)
        torch.cuda.synchronize()
        zr().zr_reduce_scatter_frags(fp, sizes, N, [g.ptr() for g in by_call], **kw)
        plan.launch()
        torch.cuda.synchronize()
        for r in range(K):
            assert np.array_equal(bits(by_plan[r].get()), bits(by_call[r].get())), f"launch {tag} rank {r}"
            assert by_plan[r].guards_intact()
    plan.close()


def test_reduce_scatter_frags_equals_gpu_flatten_then_rs():
    import torch
    from synth import workloads as W
    K = 8
    sizes = W.flatten8_numels()
    N = -(-sum(sizes) // K) * K
    C = N // K
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(K)]
    for r in range(K):
        for p in range(len(sizes)):
            synth.dev_normal_bf16(frags[r][p], SEED + 5, r * 64 + p, 0, 1e-3)
    buckets = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    a = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    b = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    zr().zr_flatten_bucket(frags, sizes, buckets, N)
    zr().zr_reduce_scatter_avg(buckets, N, a, chunk_shift=1, average=True)
    zr().zr_reduce_scatter_frags(frags, sizes, N, b, chunk_shift=1, average=True)
    torch.cuda.synchronize()
    for r in range(K):
        assert torch.equal(a[r].view(torch.int32), b[r].view(torch.int32))


def test_zero_sized_calls_enqueue_nothing():
    import torch
    m = zr()
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    m.zr_reduce_scatter_avg([t] * 4, 0, [t] * 4)
    m.zr_allreduce([t] * 4, [t] * 4, 0)
    m.zr_all_gather([t] * 4, [t] * 4, [])
    m.zr_flatten_bucket([[] for _ in range(4)], [], [t] * 4, 0)
    torch.cuda.synchronize()


# Output offsets (elements) across the 16 KiB blocks the vector tiles align
# to: the head before the first tile runs from nothing to a whole block plus
# a line, and can exceed a small chunk.
HEAD_CASES = [
    # K, N, out_bf16, out offset
    (8, 8 * 40000 + 13, False, 0),
    (8, 8 * 40000 + 13, False, 4),
    (8, 8 * 40000 + 13, False, 1000),
    (8, 8 * 40000 + 13, False, 4092),
    (8, 8 * 40000 + 13, True, 8188),
    (8, 8 * 40000 + 13, True, 3000),
    (8, 8 * 3000 + 5, False, 2048),      # odd C: only some chunks take the vector path
    (8, 8 * 40000 - 5, False, 1000),     # C a multiple of 4: every chunk vector, padded tail
    (8, 8 * 1000 - 3, False, 2048),      # heads longer than the chunk (and its padding)
    (8, 8 * 1000 - 3, True, 100),
    (5, 5 * 20000 + 3, False, 777),
    (64, 64 * 9000 + 1, True, 5000),
    (8, 8 * 300000 + 13, False, 2500),   # four-slice tiles
]


@pytest.mark.parametrize("K,N,out_bf16,out_off", HEAD_CASES)
def test_reduce_scatter_heads_across_output_blocks(K, N, out_bf16, out_off):
    import torch
    case = K * 7919 + N + out_off
    xs = make_inputs(K, N, True, case)
    C = -(-N // K)
    ins = [Guarded(N, torch.bfloat16, 0, xs[r]) for r in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), out_off) for _ in range(K)]
    zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs], chunk_shift=1,
                               average=True, in_dtype=torch.bfloat16, out_dtype=torch_dt(out_bf16))
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(xs, N, np.uint16 if out_bf16 else np.float32, shift=1, average=True)
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()


@pytest.mark.parametrize("K,sizes,out_bf16,out_off", [
    (8, [5000, 3, 70000, 40001], False, 1000),
    (8, [5000, 3, 70000, 40001], True, 8000),
    (8, [30001, 1, 2], False, 4096 - 3),
    (5, [12345, 67890], False, 333),
    (8, [1000000, 1500001, 3], False, 2500),   # four-slice tiles
])
def test_reduce_scatter_frags_heads_across_output_blocks(K, sizes, out_bf16, out_off):
    import torch
    total = sum(sizes)
    N = total + 7
    C = -(-N // K)
    frags_np = [[synth.host_normal_bf16(SEED + 91, r * 64 + p, 0, n, 1.0, 0.01, 1e4)
                 for p, n in enumerate(sizes)] for r in range(K)]
    frags = [[Guarded(n, torch.bfloat16, 0, frags_np[r][p]) for p, n in enumerate(sizes)]
             for r in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), out_off) for _ in range(K)]
    zr().zr_reduce_scatter_frags([[g.ptr() for g in row] for row in frags], sizes, N,
                                 [g.ptr() for g in outs], chunk_shift=1, average=True,
                                 in_dtype=torch.bfloat16, out_dtype=torch_dt(out_bf16))
    torch.cuda.synchronize()
    want = oracle.reduce_scatter(oracle.flatten(frags_np, sizes, N), N,
                                 np.uint16 if out_bf16 else np.float32, shift=1, average=True)
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()
