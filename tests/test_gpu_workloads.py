"""The five workloads, and the discrete path on one layer, at their full sizes,
in the launch configuration the benchmark uses, checked against the CPU oracle
on sampled outputs (the oracle computes each sampled output from the same
seeded inputs), on every output where the host can afford the oracle (the
ZeRO-2 partitions, the K=64 all-reduce), and by properties that hold at any
size (every rank identical after all-reduce, gathered parameters equal to the
generator's weights, every partition element written).

Small workloads (the 4-rank ring example and the 64-fragment bucket) are
checked in full.
"""
import gc
import sys
import threading

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_util import bits, down16, up16

pytestmark = pytest.mark.gpu


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


THREADS = 16  # host threads for whole-output oracle checks


def oracle_rs_threaded(xs, N, shift, old=None):
    """The oracle's reduce-scatter + /K of a whole bucket into fp32, split over
    host threads by chunk offset; with `old` (the K partitions before the
    call) it accumulates into them."""
    K = len(xs)
    C = -(-N // K)
    if old is None:
        outs = [np.empty(C, dtype=np.float32) for _ in range(K)]
    else:
        outs = [np.array(o, dtype=np.float32) for o in old]

    def work(i):
        oracle.reduce_scatter(xs, N, np.float32, shift=shift, average=True,
                              o_range=(i * C // THREADS, (i + 1) * C // THREADS), out=outs,
                              accumulate=old is not None)
    th = [threading.Thread(target=work, args=(i,)) for i in range(THREADS)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    return outs


def oracle_fold_bf16_threaded(xh, start):
    """The oracle's ring-order fold of every column of xh [K, n] (bf16 bits)
    from rank `start`, rounded once to bf16; widening, fold and rounding are
    split over host threads by column."""
    n = xh.shape[1]
    out = np.empty(n, dtype=np.uint16)

    def work(i):
        a, b = i * n // THREADS, (i + 1) * n // THREADS
        xf = oracle.bf16_to_f32(np.ascontiguousarray(xh[:, a:b]))
        out[a:b] = oracle.f32_to_bf16(oracle.fold_points(xf, np.full(b - a, start)))
    th = [threading.Thread(target=work, args=(i,)) for i in range(THREADS)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    return out


# ------------------------------------------------------------- ring4 (cfg 1)
def test_ring4_allreduce_exact_and_placement():
    import torch
    K, N = W.RING4["K"], W.RING4["N"]
    seed = W.seed_of(1)
    xs = [synth.host_uniform_int_f32(seed, r, 0, N, W.RING4["lo"], W.RING4["hi"]) for r in range(K)]
    total = np.sum(np.stack(xs).astype(np.int64), axis=0)
    dev = [torch.from_numpy(x).cuda() for x in xs]
    # reduce-scatter: rank r holds chunk (r+1) mod K, the exact integer sums
    C = N // K
    outs = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    zr().zr_reduce_scatter_avg(dev, N, outs, chunk_shift=1, average=False)
    for fused in (True, False):
        ar = [torch.empty(N, dtype=torch.float32, device="cuda") for _ in range(K)]
        scratch = None if fused else torch.empty(N, dtype=torch.float32, device="cuda")
        zr().zr_allreduce(dev, ar, N, average=False, fused=fused, scratch=scratch)
        torch.cuda.synchronize()
        for r in range(K):
            assert np.array_equal(ar[r].cpu().numpy(), total.astype(np.float32))
    for r in range(K):
        j = (r + 1) % K
        assert np.array_equal(outs[r].cpu().numpy(), total[j * C:(j + 1) * C].astype(np.float32))
    # the device generator reproduces the host inputs
    d = torch.empty(N, dtype=torch.float32, device="cuda")
    for r in range(K):
        synth.dev_uniform_int_f32(d, seed, r, 0, W.RING4["lo"], W.RING4["hi"])
        torch.cuda.synchronize()
        assert np.array_equal(d.cpu().numpy(), xs[r])


# ---------------------------------------------------------- flatten8 (cfg 2)
def test_flatten8_bucket_then_reduce_scatter_exact():
    import torch
    K, F = W.FLATTEN8["K"], W.FLATTEN8["n_frag"]
    seed, sigma = W.seed_of(2), W.FLATTEN8["sigma"]
    sizes = W.flatten8_numels(F)
    total = sum(sizes)
    P = -(-total // K) * K
    frags_np = [[synth.host_normal_bf16(seed, W.flatten8_frag_stream(r, p), 0, n, sigma)
                 for p, n in enumerate(sizes)] for r in range(K)]
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
             for _ in range(K)]
    for r in range(K):
        for p, n in enumerate(sizes):
            synth.dev_normal_bf16(frags[r][p], seed, W.flatten8_frag_stream(r, p), 0, sigma)
    buckets = [torch.empty(P, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    C = P // K
    parts = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    zr().zr_flatten_bucket(frags, sizes, buckets, P)
    zr().zr_reduce_scatter_avg(buckets, P, parts, chunk_shift=1, average=True)
    torch.cuda.synchronize()
    want_b = oracle.flatten(frags_np, sizes, P)
    want_p = oracle.reduce_scatter(want_b, P, np.float32, shift=1, average=True)
    for r in range(K):
        assert np.array_equal(down16(buckets[r]), want_b[r])
        assert np.array_equal(bits(parts[r].cpu().numpy()), bits(want_p[r]))
    say(f"flatten8: {F} fragments, {total} elements, padded to {P}")


# -------------------------------------------------------- zero2_grad (cfg 3)
def sample_offsets(rng, C, m):
    o = rng.integers(0, C, size=m)
    return np.unique(np.concatenate([o, [0, 1, 7, 8, C // 2, C - 9, C - 8, C - 2, C - 1]]))


def test_zero2_grad_sync_full_size_sampled():
    import torch
    from gradient_sync_zr_amd.steps import Zero2GradSync
    cfg = W.ZERO2
    K, N, bucket, sigma = cfg["K"], cfg["N_total"], cfg["bucket"], cfg["sigma"]
    seed = W.seed_of(3)
    say(f"zero2: allocating {K} x {N} bf16 grads")
    grads = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for r in range(K):
        synth.dev_normal_bf16(grads[r], seed, r, 0, sigma)
    buckets = W.zero2_buckets(N, bucket)
    P = sum(-(-n // K) for _, n in buckets)
    parts = [torch.empty(P, dtype=torch.float32, device="cuda") for _ in range(K)]
    for p in parts:
        p.view(torch.int32).fill_(-1)  # NaN sentinel: every element must be written
    red = torch.cuda.Stream()
    sync = Zero2GradSync(grads, parts, bucket, chunk_shift=cfg["shift"], average=True,
                         reduction_stream=red)
    sync.step()
    torch.cuda.synchronize()
    say("zero2: step done, checking")
    for p in parts:
        assert not bool(torch.isnan(p).any())
    rng = np.random.default_rng(3)
    poff = 0
    for (start, n) in buckets:
        Cb = -(-n // K)
        offs = sample_offsets(rng, Cb, 3000)
        M = offs.size
        # the sampled outputs form a small reduce-scatter of their own: chunk j
        # of the small problem holds, at position m, the inputs of offset offs[m]
        # of chunk j of this bucket
        X = np.zeros((K, K * M), dtype=np.uint16)
        for j in range(K):
            g = j * Cb + offs
            ok = g < n
            for r in range(K):
                vals = synth.host_points_normal_bf16(seed, np.full(M, r), start + np.minimum(g, n - 1),
                                                     sigma)
                X[r, j * M:(j + 1) * M] = np.where(ok, vals, 0)
        want = oracle.reduce_scatter([X[r] for r in range(K)], K * M, np.float32, shift=1,
                                     average=True)
        idx = torch.from_numpy(poff + offs).cuda()
        for q in range(K):
            got = parts[q].index_select(0, idx).cpu().numpy()
            assert np.array_equal(bits(got), bits(want[q])), f"bucket at {start}, rank {q}"
        poff += Cb
    # every partition element, bucket by bucket, against the oracle on the
    # same resident inputs copied to the host
    poff = 0
    for (start, n) in buckets:
        Cb = -(-n // K)
        xs = [grads[r][start:start + n].view(torch.int16).cpu().numpy().view(np.uint16)
              for r in range(K)]
        want = oracle_rs_threaded(xs, n, cfg["shift"])
        for q in range(K):
            got = parts[q][poff:poff + Cb].cpu().numpy()
            assert np.array_equal(bits(got), bits(want[q])), f"whole bucket at {start}, rank {q}"
        del xs, want
        poff += Cb
    say("zero2: every partition element bit-exact against the oracle")
    # gradient accumulation at full size: a second micro-step with new
    # gradients adds its averages to the partitions; every element against
    # the oracle's accumulating reduce-scatter
    first = [p.cpu().numpy() for p in parts]
    for r in range(K):
        synth.dev_normal_bf16(grads[r], seed + 0x100, r, 0, sigma)
    sync.step(micro_step=1)
    torch.cuda.synchronize()
    poff = 0
    for (start, n) in buckets:
        Cb = -(-n // K)
        xs = [grads[r][start:start + n].view(torch.int16).cpu().numpy().view(np.uint16)
              for r in range(K)]
        want = oracle_rs_threaded(xs, n, cfg["shift"], old=[f[poff:poff + Cb] for f in first])
        for q in range(K):
            got = parts[q][poff:poff + Cb].cpu().numpy()
            assert np.array_equal(bits(got), bits(want[q])), f"accumulate bucket at {start}, rank {q}"
        del xs, want
        poff += Cb
    del first
    sync.close()
    say("zero2: sampled outputs bit-exact; accumulation micro-step bit-exact on every element")


# ------------------------------------------------ discrete path, one layer
def test_frags_layer_discrete_full_size():
    """The discrete reduce-scatter over one layer's seven gradients per rank,
    at full size: sampled outputs against the oracle from the host generator,
    every output against the oracle's flatten + reduce-scatter of the
    fragments copied to the host, every output equal to flatten + contiguous
    reduce-scatter on the GPU, every element written."""
    import torch
    cfg = W.FRAGS_LAYER
    K, sigma, shift = cfg["K"], cfg["sigma"], cfg["shift"]
    seed = W.seed_of(cfg["seed_cfg"])
    sizes = W.frags_layer_numels()
    N = sum(sizes)
    C = -(-N // K)
    say(f"frags_layer: {K} x {len(sizes)} fragments, {N} elements per rank")
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(K)]
    for r in range(K):
        for p in range(len(sizes)):
            synth.dev_normal_bf16(frags[r][p], seed, W.frags_layer_stream(r, p), 0, sigma)
    parts = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    for p in parts:
        p.view(torch.int32).fill_(-1)  # NaN sentinel: every element must be written
    zr().zr_reduce_scatter_frags(frags, sizes, N, parts, chunk_shift=shift, average=True,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    for p in parts:
        assert not bool(torch.isnan(p).any())
    # sampled outputs: virtual index g lies in fragment p at local offset g - start_p
    starts = np.cumsum([0] + sizes)
    offs = sample_offsets(np.random.default_rng(6), C, 3000)
    M = offs.size
    X = np.zeros((K, K * M), dtype=np.uint16)
    for j in range(K):
        g = j * C + offs
        ok = g < N
        gg = np.minimum(g, N - 1)
        frag = np.searchsorted(starts, gg, side="right") - 1
        for r in range(K):
            streams = np.array([W.frags_layer_stream(r, int(f)) for f in frag])
            vals = synth.host_points_normal_bf16(seed, streams, gg - starts[frag], sigma)
            X[r, j * M:(j + 1) * M] = np.where(ok, vals, 0)
    want = oracle.reduce_scatter([X[r] for r in range(K)], K * M, np.float32, shift=shift,
                                 average=True)
    idx = torch.from_numpy(offs).cuda()
    for q in range(K):
        got = parts[q].index_select(0, idx).cpu().numpy()
        assert np.array_equal(bits(got), bits(want[q])), f"rank {q}"
    # whole outputs against the oracle: the fragments copied to the host,
    # flattened into padded buckets and reduced there
    fh = [[down16(f) for f in frags[r]] for r in range(K)]
    bh = oracle.flatten(fh, sizes, K * C)
    del fh
    want = oracle_rs_threaded(bh, N, shift)
    del bh
    for q in range(K):
        assert np.array_equal(bits(parts[q].cpu().numpy()), bits(want[q])), f"rank {q}"
    del want
    say("frags_layer: every output bit-exact against the oracle")
    # whole outputs: the same as flattening into a bucket and reducing it
    buckets = [torch.empty(K * C, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    zr().zr_flatten_bucket(frags, sizes, buckets, K * C)
    del frags
    ref = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    zr().zr_reduce_scatter_avg(buckets, K * C, ref, chunk_shift=shift, average=True)
    torch.cuda.synchronize()
    for q in range(K):
        assert torch.equal(parts[q].view(torch.int32), ref[q].view(torch.int32)), f"rank {q}"
    say("frags_layer: sampled outputs bit-exact; equal to flatten + reduce-scatter")


# ---------------------------------------------------------- zero3_ag (cfg 4)
def test_zero3_allgather_full_size():
    import torch
    from gradient_sync_zr_amd.steps import Zero3Gather
    cfg = W.ZERO3
    K, sigma, shift = cfg["K"], cfg["sigma"], cfg["shift"]
    seed = W.seed_of(4)
    ps = W.llama_like_params()
    numels = [p.numel for p in ps]
    shard_numel = sum(-(-n // K) for n in numels)
    full_numel = sum(numels)
    say(f"zero3: {len(ps)} params, shards {shard_numel}, full {full_numel}")
    shards = [torch.zeros(shard_numel, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    fulls = [torch.empty(full_numel, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for f in fulls:
        f.view(torch.int16).fill_(-1)
    soff = 0
    for p, n in enumerate(numels):
        C = -(-n // K)
        for r in range(K):
            j = (r + shift) % K      # the chunk rank r holds
            cnt = max(0, min(C, n - j * C))
            if cnt:
                synth.dev_normal_bf16(shards[r][soff:soff + cnt], seed, p, j * C, sigma)
        soff += C
    gather = Zero3Gather(shards, fulls, numels, cfg["prefetch_bytes"] // cfg["elem_bytes"],
                         chunk_shift=shift)
    assert len(gather.buckets) == 162
    gather.step()
    torch.cuda.synchronize()
    say("zero3: gathered, comparing with the generator's weights")
    tmp = torch.empty(max(numels), dtype=torch.bfloat16, device="cuda")
    for p, (so, fo, n) in enumerate(gather.param_offsets):
        synth.dev_normal_bf16(tmp[:n], seed, p, 0, sigma)
        w = tmp[:n].view(torch.int16)
        for r in range(K):
            assert torch.equal(fulls[r][fo:fo + n].view(torch.int16), w), f"param {p} rank {r}"
    # host twin on sampled points (independent of the device generator)
    rng = np.random.default_rng(4)
    pi = rng.integers(0, len(ps), size=4000)
    gi = np.array([rng.integers(0, numels[p]) for p in pi], dtype=np.int64)
    want = synth.host_points_normal_bf16(seed, pi, gi, sigma)
    fo = np.array([gather.param_offsets[p][1] for p in pi], dtype=np.int64)
    for r in range(K):
        got = down16(fulls[r].index_select(0, torch.from_numpy(fo + gi).cuda()))
        assert np.array_equal(got, want)
    # the oracle's all-gather on a sampled sub-problem: one bucket's segments,
    # shards copied back to the host
    segs = gather.buckets[1]
    lo = min(s[0] for s in segs)
    hi = max(s[0] + -(-s[2] // K) for s in segs)
    sh_np = [down16(shards[r][lo:hi]) for r in range(K)]
    flo = min(s[1] for s in segs)
    fhi = max(s[1] + s[2] for s in segs)
    f_np = [np.zeros(fhi - flo, dtype=np.uint16) for _ in range(K)]
    oracle.all_gather(sh_np, f_np, [(s[0] - lo, s[1] - flo, s[2]) for s in segs], shift)
    for r in range(K):
        assert np.array_equal(down16(fulls[r][flo:fhi]), f_np[r])
    say("zero3: all 8 ranks hold every parameter, bit-exact")


# -------------------------------------------------------- allreduce64 (cfg 5)
def test_allreduce64_full_size_fused_and_composed():
    import torch
    cfg = W.ALLREDUCE64
    K, N = cfg["K"], cfg["N"]
    sigma, p_out, mag = cfg["sigma"], cfg["outlier_p"], cfg["outlier_mag"]
    seed = W.seed_of(5)
    C = -(-N // K)
    stride = -(-N // 128) * 128
    say(f"allreduce64: K={K} N={N} C={C}, {K * stride * 2 / 1e9:.1f} GB")
    buf = torch.empty(K * stride, dtype=torch.bfloat16, device="cuda")
    ranks = [buf[r * stride:r * stride + N] for r in range(K)]

    # sampled positions: random, every chunk boundary, and the end
    rng = np.random.default_rng(5)
    pts = [rng.integers(0, N, size=20000)]
    for j in range(1, K):
        pts.append(np.arange(j * C - 9, j * C + 9))
    pts.append(np.arange(N - 17, N))
    g = np.unique(np.concatenate(pts))
    g = g[(g >= 0) & (g < N)]
    # expected: a small all-reduce whose chunk j holds the sampled points of
    # chunk j (same ring start rank), computed by the oracle
    chunk = g // C
    M = int(np.bincount(chunk, minlength=K).max())
    X = np.zeros((K, K * M), dtype=np.uint16)
    slot = np.full(g.size, -1)
    for j in range(K):
        sel = np.nonzero(chunk == j)[0]
        slot[sel] = j * M + np.arange(sel.size)
    for r in range(K):
        X[r, slot] = synth.host_points_normal_bf16(seed, np.full(g.size, r), g, sigma, p_out, mag)
    want = oracle.allreduce([X[r] for r in range(K)], K * M, average=False)[0][slot]
    idx = torch.from_numpy(g).cuda()
    view = buf.view(K, stride)

    fused_r0 = None
    for fused in (True, False):
        for r in range(K):
            synth.dev_normal_bf16(ranks[r], seed, r, 0, sigma, p_out, mag)
        scratch = None if fused else torch.empty(K * C, dtype=torch.bfloat16, device="cuda")
        zr().zr_allreduce(ranks, ranks, N, average=False, fused=fused, scratch=scratch)
        torch.cuda.synchronize()
        say(f"allreduce64: fused={fused} done, checking")
        got = down16(view.index_select(1, idx))
        for r in range(K):
            assert np.array_equal(got[r], want), f"fused={fused} rank {r}"
        r0 = ranks[0].view(torch.int16)
        for r in range(1, K):
            assert torch.equal(ranks[r].view(torch.int16), r0), f"rank {r} differs from rank 0"
        del scratch
        if fused:
            fused_r0 = r0.clone()
            # every output element against the oracle, a chunk at a time: the
            # chunk's 64 input slices are regenerated on the device (the
            # in-place all-reduce overwrote them) and folded on the host
            x = torch.empty((K, C), dtype=torch.bfloat16, device="cuda")
            for j in range(K):
                n = min(C, N - j * C)
                for r in range(K):
                    synth.dev_normal_bf16(x[r, :n], seed, r, j * C, sigma, p_out, mag)
                xh = x[:, :n].view(torch.int16).cpu().numpy().view(np.uint16)
                expect = oracle_fold_bf16_threaded(xh, j)
                del xh
                assert np.array_equal(down16(ranks[0][j * C:j * C + n]), expect), f"chunk {j}"
                if j % 16 == 15 or j == K - 1:
                    say(f"allreduce64: chunks 0..{j} bit-exact against the oracle")
            del x
        else:
            assert torch.equal(r0, fused_r0), "composed all-reduce differs from the fused one"
    say("allreduce64: every output bit-exact against the oracle, all 64 ranks identical, "
        "fused == composed on every element")
