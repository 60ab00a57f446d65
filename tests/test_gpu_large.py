"""Single calls past 2^31 elements per rank: the kernels' 64-bit offsets.

Every rank buffer here holds more than 2^31 bf16 elements (over 4 GiB), so the global index and the
input byte offsets both pass 32 bits inside one call. The checks are:
  - the reduce-scatter and the discrete path: sampled outputs against the oracle, computed from the
    same seeded inputs, with the samples set densely around the index 2^31 and at the chunk ends;
    every partition element must also be written;
  - the fused all-reduce (in place): sampled outputs of rank 0 against the oracle, and every rank
    identical to rank 0 on every element;
  - the all-gather: every element of every rank's full buffer equal to the unsharded tensor. A second
    segment starts past 2^31 in the full buffers;
  - the flatten: every element of every bucket equal to its fragment, and zero padding after them;
  - ranks whose views sit in different phases: the reduce-scatter and the fused all-reduce, sampled
    as above.
"""
import gc
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits

pytestmark = pytest.mark.gpu

SEED = 0x5A5200B0
BIG = (1 << 31) + (1 << 21) + 13   # elements per rank: past 2^31, not a multiple of 8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def free_memory():
    yield
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def zr():
    import gradient_sync_zr_amd as m
    return m


def offsets(rng, C, lo_edge, m=1500):
    """Sorted distinct chunk offsets in [0, C): random ones, the chunk's first and last 8, and 64
    around `lo_edge` (the offset of global index 2^31 in this chunk, if it falls inside)."""
    pick = [rng.integers(0, C, m), np.arange(8), np.arange(C - 8, C)]
    if 0 <= lo_edge < C:
        pick.append(np.clip(np.arange(lo_edge - 32, lo_edge + 32), 0, C - 1))
    return np.unique(np.concatenate(pick)).astype(np.int64)


def sampled_rs_want(K, N, C, value_at, rng, shift, average):
    """(per-chunk offsets, the oracle's partitions over them): the sampled outputs form a small
    reduce-scatter of their own, whose chunk j holds at position m the inputs of offset offs[m] of
    chunk j here (zero where the global index is padding)."""
    offs = [offsets(rng, C, (1 << 31) - j * C) for j in range(K)]
    M = max(o.size for o in offs)
    offs = [np.concatenate([o, np.full(M - o.size, o[-1])]) for o in offs]  # pad by repeating
    X = np.zeros((K, K * M), dtype=np.uint16)
    for j in range(K):
        g = j * C + offs[j]
        ok = g < N
        for r in range(K):
            X[r, j * M:(j + 1) * M] = np.where(ok, value_at(r, np.minimum(g, N - 1)), 0)
    want = oracle.reduce_scatter([X[r] for r in range(K)], K * M, np.float32, shift=shift,
                                 average=average)
    return offs, want, M


def test_reduce_scatter_past_2e31():
    _reduce_scatter_past_2e31(8, BIG)


@pytest.mark.parametrize("K", [8, 16])
def test_reduce_scatter_vector_path_past_2e31(K):
    """Chunks on the quad grid (C a multiple of 4, N three short of K*C), so
    every chunk takes the contiguous kernel's vector path: at K = 8 the static
    one-slice kernel, at K = 16 the generic one. (BIG's chunks start off the
    grid, which routes the call through the discrete kernel.)"""
    C = -(-(1 << 31) // K)
    C += (-C) % 4 + 4
    _reduce_scatter_past_2e31(K, K * C - 3)


def _reduce_scatter_past_2e31(K, N):
    import torch
    shift = 1
    C = -(-N // K)
    say(f"large rs: K={K} N={N}")
    xs = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for r in range(K):
        synth.dev_normal_bf16(xs[r], SEED, r, 0, 1.0, 0.01, 1e4)
    outs = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    for o in outs:
        o.view(torch.int32).fill_(-1)  # NaN sentinel: every element must be written
    zr().zr_reduce_scatter_avg([x.data_ptr() for x in xs], N, [o.data_ptr() for o in outs],
                               chunk_shift=shift, average=True, in_dtype=torch.bfloat16,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    for o in outs:
        assert not bool(torch.isnan(o).any())
    rng = np.random.default_rng(31)

    def value_at(r, g):
        return synth.host_points_normal_bf16(SEED, np.full(g.size, r), g, 1.0, 0.01, 1e4)

    offs, want, M = sampled_rs_want(K, N, C, value_at, rng, shift, True)
    for q in range(K):
        j = (q + shift) % K
        got = outs[q].index_select(0, torch.from_numpy(offs[j]).cuda()).cpu().numpy()
        assert np.array_equal(bits(got), bits(want[q][:M])), f"rank {q}"
    say("large rs: sampled outputs bit-exact")


def test_reduce_scatter_frags_past_2e31():
    import torch
    K, shift = 8, 1
    sizes = [(1 << 31) + 5, 1000, 3]
    N = sum(sizes) + 7
    C = -(-N // K)
    cuts = np.cumsum([0] + sizes)
    say(f"large frags: K={K} sizes={sizes}")
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(K)]
    for r in range(K):
        for p in range(len(sizes)):
            synth.dev_normal_bf16(frags[r][p], SEED + 1, r * 16 + p, 0, 1.0, 0.01, 1e4)
    outs = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    for o in outs:
        o.view(torch.int32).fill_(-1)
    zr().zr_reduce_scatter_frags([[f.data_ptr() for f in row] for row in frags], sizes, N,
                                 [o.data_ptr() for o in outs], chunk_shift=shift, average=True,
                                 in_dtype=torch.bfloat16, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for o in outs:
        assert not bool(torch.isnan(o).any())
    rng = np.random.default_rng(32)

    def value_at(r, g):
        # index g of the virtual bucket: fragment p at local index g - cuts[p], zero past the last
        p = np.searchsorted(cuts, g, side="right") - 1
        v = np.zeros(g.size, dtype=np.uint16)
        inside = p < len(sizes)
        pi, gi = p[inside], g[inside]
        v[inside] = synth.host_points_normal_bf16(SEED + 1, r * 16 + pi, gi - cuts[pi], 1.0, 0.01,
                                                  1e4)
        return v

    offs, want, M = sampled_rs_want(K, N, C, value_at, rng, shift, True)
    for q in range(K):
        j = (q + shift) % K
        got = outs[q].index_select(0, torch.from_numpy(offs[j]).cuda()).cpu().numpy()
        assert np.array_equal(bits(got), bits(want[q][:M])), f"rank {q}"
    say("large frags: sampled outputs bit-exact")


def test_allreduce_past_2e31():
    import torch
    K, N = 8, (1 << 31) + 77
    C = -(-N // K)
    say(f"large ar: K={K} N={N}")
    bufs = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for r in range(K):
        synth.dev_normal_bf16(bufs[r], SEED + 2, r, 0, 1.0, 0.01, 1e4)
    zr().zr_allreduce([b.data_ptr() for b in bufs], [b.data_ptr() for b in bufs], N, average=False,
                      dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for r in range(1, K):
        assert torch.equal(bufs[r].view(torch.int16), bufs[0].view(torch.int16)), f"rank {r}"
    rng = np.random.default_rng(33)
    g = np.unique(np.concatenate([
        rng.integers(0, N, 20000), np.arange(N - 16, N), np.arange((1 << 31) - 64, (1 << 31) + 64),
        np.concatenate([np.arange(j * C - 4, j * C + 4) for j in range(1, K)])])).astype(np.int64)
    xs = np.stack([synth.host_points_normal_bf16(SEED + 2, np.full(g.size, r), g, 1.0, 0.01, 1e4)
                   for r in range(K)])
    start = g // C   # each index folds from the first rank of its chunk
    want = oracle.f32_to_bf16(oracle.fold_points(oracle.bf16_to_f32(xs), start))
    got = bufs[0].view(torch.int16).index_select(0, torch.from_numpy(g).cuda()).cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want)
    say("large ar: sampled outputs bit-exact, all ranks identical")


def test_all_gather_past_2e31():
    import torch
    K, shift = 8, 0
    n0, n1 = (1 << 31) + 4099, 777
    C0, C1 = -(-n0 // K), -(-n1 // K)
    say(f"large ag: K={K} segments {n0}, {n1}")
    w = torch.empty(n0 + n1, dtype=torch.bfloat16, device="cuda")
    synth.dev_normal_bf16(w, SEED + 3, 0, 0, 0.02)
    shards = [torch.zeros(C0 + C1, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for q in range(K):
        j = (q + shift) % K
        for (off, n, C, soff) in ((0, n0, C0, 0), (n0, n1, C1, C0)):
            lo, hi = j * C, min((j + 1) * C, n)
            if hi > lo:
                shards[q][soff:soff + hi - lo].copy_(w[off + lo:off + hi])
    fulls = [torch.empty(n0 + n1, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for f in fulls:
        f.view(torch.int16).fill_(-1)
    zr().zr_all_gather([s.data_ptr() for s in shards], [f.data_ptr() for f in fulls],
                       [(0, 0, n0), (C0, n0, n1)], chunk_shift=shift, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for r in range(K):
        assert torch.equal(fulls[r].view(torch.int16), w.view(torch.int16)), f"rank {r}"
    say("large ag: every element of every rank equals the unsharded tensor")


def test_flatten_past_2e31():
    import torch
    K = 4
    sizes = [5, (1 << 31) + 3, 1001]
    total = sum(sizes)
    padded = total + 9
    say(f"large flatten: K={K} sizes={sizes}")
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(K)]
    for r in range(K):
        for p in range(len(sizes)):
            synth.dev_normal_bf16(frags[r][p], SEED + 4, r * 16 + p, 0, 1e-3)
    buckets = [torch.empty(padded, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for b in buckets:
        b.view(torch.int16).fill_(-1)
    zr().zr_flatten_bucket([[f.data_ptr() for f in row] for row in frags], sizes,
                           [b.data_ptr() for b in buckets], padded, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for r in range(K):
        off = 0
        for p, n in enumerate(sizes):
            assert torch.equal(buckets[r][off:off + n].view(torch.int16),
                               frags[r][p].view(torch.int16)), f"rank {r} fragment {p}"
            off += n
        assert bool((buckets[r][total:].view(torch.int16) == 0).all()), f"rank {r} padding"
    say("large flatten: every bucket element equals its fragment; padding zero")


def test_ranks_in_mixed_phases_past_2e31():
    # rank r's views start r mod 4 elements into their allocations: the reduce-scatter (through
    # the discrete path's aligned-pair folds) and the fused all-reduce (aligned pairs and LDS-staged
    # stores) past 2^31 elements per rank, sampled against the oracle
    import torch
    K, N, shift = 4, BIG, 1
    C = -(-N // K)
    say(f"large mixed phases: K={K} N={N}")
    base = [torch.empty(N + 4, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    xs = [base[r][r % 4:r % 4 + N] for r in range(K)]
    for r in range(K):
        synth.dev_normal_bf16(xs[r], SEED + 5, r, 0, 1.0, 0.01, 1e4)
    obase = [torch.empty(C + 4, dtype=torch.float32, device="cuda") for _ in range(K)]
    outs = [obase[r][(r + 1) % 4:(r + 1) % 4 + C] for r in range(K)]
    for o in outs:
        o.view(torch.int32).fill_(-1)
    zr().zr_reduce_scatter_avg([x.data_ptr() for x in xs], N, [o.data_ptr() for o in outs],
                               chunk_shift=shift, average=True, in_dtype=torch.bfloat16,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    for o in outs:
        assert not bool(torch.isnan(o).any())
    rng = np.random.default_rng(35)

    def value_at(r, g):
        return synth.host_points_normal_bf16(SEED + 5, np.full(g.size, r), g, 1.0, 0.01, 1e4)

    offs, want, M = sampled_rs_want(K, N, C, value_at, rng, shift, True)
    for q in range(K):
        j = (q + shift) % K
        got = outs[q].index_select(0, torch.from_numpy(offs[j]).cuda()).cpu().numpy()
        assert np.array_equal(bits(got), bits(want[q][:M])), f"rs rank {q}"
    say("large mixed phases: reduce-scatter sampled outputs bit-exact")
    del obase, outs
    gc.collect()
    torch.cuda.empty_cache()
    # the fused all-reduce in place on the same views (sum, no average)
    zr().zr_allreduce([x.data_ptr() for x in xs], [x.data_ptr() for x in xs], N, average=False,
                      dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for r in range(1, K):
        assert torch.equal(xs[r].view(torch.int16), xs[0].view(torch.int16)), f"ar rank {r}"
    g = np.unique(np.concatenate([
        rng.integers(0, N, 20000), np.arange(N - 16, N), np.arange((1 << 31) - 64, (1 << 31) + 64),
        np.concatenate([np.arange(j * C - 4, j * C + 4) for j in range(1, K)])])).astype(np.int64)
    pts = np.stack([value_at(r, g) for r in range(K)])
    want_ar = oracle.f32_to_bf16(oracle.fold_points(oracle.bf16_to_f32(pts), g // C))
    got = xs[0].view(torch.int16).index_select(0, torch.from_numpy(g).cuda()).cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want_ar)
    say("large mixed phases: all-reduce sampled outputs bit-exact, all ranks identical")
