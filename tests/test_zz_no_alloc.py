"""The allocation-free discrete reduce-scatter against the one-shot call.

zr_reduce_scatter_frags_noalloc stages a table that does not fit one
kernel-argument block in the library's file-scope device array instead of a
caller's workspace. Two calls in a row, the second with a smaller table (and
other K), must equal zr_reduce_scatter_frags (no workspace: argument
launches) bit for bit, and the oracle's flatten followed by its
reduce-scatter; a table beyond the array is refused with nothing written.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Guarded, bits

pytestmark = pytest.mark.gpu

SEED = 0x5A5200D0


def zr():
    import gradient_sync_zr_amd as m
    return m


def case(K, F, seed, hi=3000):
    """F fragments per rank, views into one buffer per rank at varying quad
    phases; outputs for both entry points."""
    import torch
    rng = np.random.default_rng(seed)
    sizes = [int(x) for x in rng.integers(1, hi, size=F)]
    gaps = [int(x) for x in rng.integers(0, 8, size=F)]
    frags_np = [[synth.host_normal_bf16(SEED + seed, r * 4096 + p, 0, n, 1.0, 0.01, 1e4)
                 for p, n in enumerate(sizes)] for r in range(K)]
    offs, o = [], 0
    for n, g in zip(sizes, gaps):
        o += g
        offs.append(o)
        o += n
    bufs, ptrs = [], []
    for r in range(K):
        host = np.zeros(o, dtype=np.uint16)
        for p, n in enumerate(sizes):
            host[offs[p]:offs[p] + n] = frags_np[r][p]
        g = Guarded(o, torch.bfloat16, 0, host)
        bufs.append(g)
        ptrs.append([g.ptr() + 2 * offs[p] for p in range(F)])
    N = -(-sum(sizes) // K) * K + K
    return sizes, frags_np, ptrs, bufs, N


@pytest.mark.parametrize("order", [0, 2])
def test_noalloc_equals_the_one_shot_call_twice(order):
    import torch
    kw = dict(chunk_shift=1, average=True, order=order, in_dtype=torch.bfloat16,
              out_dtype=torch.float32)
    for K, F, seed in ((64, 150, 11), (8, 45, 12)):   # the second table is smaller
        assert zr().zr_workspace_bytes(K, F) > 0       # both need staging
        sizes, frags_np, fp, bufs, N = case(K, F, seed)
        C = N // K
        a = [Guarded(C, torch.float32, 0) for _ in range(K)]
        b = [Guarded(C, torch.float32, 0) for _ in range(K)]
        print(f"noalloc K={K} F={F} N={N} order={order}", flush=True)
        zr().zr_reduce_scatter_frags_noalloc(fp, sizes, N, [g.ptr() for g in a], **kw)
        zr().zr_reduce_scatter_frags(fp, sizes, N, [g.ptr() for g in b], **kw)
        torch.cuda.synchronize()
        want = oracle.reduce_scatter(oracle.flatten(frags_np, sizes, N), N, np.float32, shift=1,
                                     average=True, wire=(order == 2))
        for q in range(K):
            assert np.array_equal(bits(a[q].get()), bits(b[q].get())), f"rank {q}"
            assert np.array_equal(bits(a[q].get()), bits(want[q])), f"rank {q}"
            assert a[q].guards_intact() and bufs[q].guards_intact()


def test_noalloc_refuses_a_table_beyond_its_array():
    import torch
    K, F = 64, 2000                                    # zr_workspace_bytes > 1 MiB
    assert zr().zr_workspace_bytes(K, F) > zr().ZR_NOALLOC_TABLE_BYTES
    sizes, frags_np, fp, bufs, N = case(K, F, 13, hi=40)
    init = np.full(N // K, 3.0, dtype=np.float32)
    outs = [Guarded(N // K, torch.float32, 0, init) for _ in range(K)]
    with pytest.raises(zr().ZrError) as e:
        zr().zr_reduce_scatter_frags_noalloc(fp, sizes, N, [g.ptr() for g in outs],
                                             in_dtype=torch.bfloat16, out_dtype=torch.float32)
    assert e.value.status == zr().ZR_ERR_WORKSPACE
    torch.cuda.synchronize()
    for q in range(K):
        assert np.array_equal(outs[q].get(), init)
