"""GPU parity when the ranks' buffers sit in different phases: every rank's
view starts its own number of elements past a quad (or, for the all-gather's
full buffers, a 16-byte) boundary, so no single tile grid aligns them all.

The reduce-scatter, its discrete form and the fused all-reduce read such
ranks as aligned quad pairs joined in registers; the all-gather stages each
tile's source in LDS and shifts it per destination. Ring and wire orders must
still match the oracle bit for bit, at sizes that span several full tiles
(both tile shapes), chunk boundaries inside tiles, ragged tails, in-place
calls and accumulation; the free order must stay within its bound of the
exact sum.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Guarded, bf16_ulp, bits

pytestmark = pytest.mark.gpu

SEED = 0x5A5200D0


def zr():
    import gradient_sync_zr_amd as m
    return m


def torch_dt(is_bf16):
    import torch
    return torch.bfloat16 if is_bf16 else torch.float32


def make_inputs(K, N, bf16, case):
    xs = [synth.host_normal_bf16(SEED + case, r, 0, N, 1.0, 0.01, 1e4) for r in range(K)]
    if bf16:
        return xs
    rng = np.random.default_rng(case)
    return [oracle.bf16_to_f32(x) * (1 + rng.standard_normal(N).astype(np.float32) * 1e-3)
            for x in xs]


def quad_phase(pattern, r):
    """Element offset of rank r's view within a quad."""
    return {"r%4": r % 4, "3r+1": (3 * r + 1) % 4, "one-off": 1 if r == 2 else 0}[pattern]


RS_CASES = [
    # K, N, in_bf16, out_bf16, order (0 ring, 2 wire), in pattern, out pattern, accumulate
    (2, 2 * 30000 + 1, True, False, 0, "r%4", "r%4", False),
    (3, 3 * 40001, True, True, 0, "3r+1", "r%4", False),
    (8, 8 * 20000 + 13, True, False, 0, "r%4", "3r+1", False),      # one-slice tiles
    (8, 8 * 300000 + 13, True, False, 0, "r%4", "r%4", False),      # four-slice tiles
    (8, 8 * 300000 + 5, True, False, 0, "one-off", "r%4", True),    # one rank off, accumulate
    (8, 8 * 300000 + 5, True, True, 2, "3r+1", "3r+1", False),      # wire order
    (8, 8 * 150000 + 3, False, False, 0, "r%4", "r%4", False),      # fp32 quads: dword selects
    (8, 8 * 150000 + 3, False, True, 0, "3r+1", "one-off", True),
    (16, 16 * 100000 + 7, True, False, 0, "r%4", "r%4", False),
    (33, 33 * 20000 + 2, True, False, 2, "3r+1", "r%4", False),
    (64, 64 * 40000 + 7, True, False, 0, "r%4", "3r+1", False),
    (64, 64 * 3000 + 1, False, False, 0, "3r+1", "r%4", True),
]


@pytest.mark.parametrize("entry", ["call", "plan"])
@pytest.mark.parametrize("K,N,in_bf16,out_bf16,order,ipat,opat,acc", RS_CASES)
def test_reduce_scatter_ranks_in_mixed_phases(K, N, in_bf16, out_bf16, order, ipat, opat, acc, entry):
    import torch
    C = -(-N // K)
    xs = make_inputs(K, N, in_bf16, K * 7919 + N)
    ins = [Guarded(N, torch_dt(in_bf16), quad_phase(ipat, r), xs[r]) for r in range(K)]
    odt = np.uint16 if out_bf16 else np.float32
    rng = np.random.default_rng(N)
    init = [oracle.f32_to_bf16(rng.standard_normal(C).astype(np.float32)) if out_bf16 else
            rng.standard_normal(C).astype(np.float32) for _ in range(K)]
    outs = [Guarded(C, torch_dt(out_bf16), quad_phase(opat, r), init[r]) for r in range(K)]
    kw = dict(chunk_shift=1, average=True, order=order, accumulate=acc, in_dtype=torch_dt(in_bf16),
              out_dtype=torch_dt(out_bf16))
    if entry == "call":
        zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs], **kw)
    else:
        plan = zr().RsPlan([g.ptr() for g in ins], N, [g.ptr() for g in outs], **kw)
        plan.launch()
        plan.close()
    torch.cuda.synchronize()
    want = [x.copy() for x in init]
    oracle.reduce_scatter(xs, N, odt, shift=1, average=True, out=want, accumulate=acc,
                          wire=(order == 2))
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact() and ins[r].guards_intact()


@pytest.mark.parametrize("K,sizes,in_bf16,ws", [
    (8, [70001, 5, 1200003], True, False),
    (16, [3, 333333, 64 * 1000 + 1], True, True),
    (64, [1 + 613 * i for i in range(64)], True, True),   # one staged launch
    (64, [1 + 613 * i for i in range(64)], True, False),  # argument launches
    (4, [100000, 7, 250001], False, False),
])
def test_discrete_reduce_scatter_ranks_in_mixed_phases(K, sizes, in_bf16, ws):
    # each fragment of rank r at its own phase (r + p) % 4; partitions at 1
    import torch
    total = sum(sizes)
    N = total + 3
    C = -(-N // K)
    frags_np = [[synth.host_normal_bf16(SEED + 5, r * 4096 + p, 0, n, 1.0, 0.01, 1e4)
                 for p, n in enumerate(sizes)] for r in range(K)]
    if not in_bf16:
        frags_np = [[oracle.bf16_to_f32(h) for h in row] for row in frags_np]
    frags = [[Guarded(n, torch_dt(in_bf16), (r + p) % 4, frags_np[r][p]) for p, n in enumerate(sizes)]
             for r in range(K)]
    outs = [Guarded(C, torch.float32, 1) for _ in range(K)]
    wsb = None
    if ws:
        wsb = torch.empty(max(256, zr().zr_workspace_bytes(K, len(sizes))), dtype=torch.uint8, device="cuda")
    zr().zr_reduce_scatter_frags([[g.ptr() for g in row] for row in frags], sizes, N,
                                 [g.ptr() for g in outs], chunk_shift=1, average=True,
                                 in_dtype=torch_dt(in_bf16), out_dtype=torch.float32, workspace=wsb)
    torch.cuda.synchronize()
    bucket = oracle.flatten(frags_np, sizes, N)
    want = oracle.reduce_scatter(bucket, N, np.float32, shift=1, average=True)
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact()


AR_CASES = [
    # K, N, bf16, order, inplace, in pattern, out pattern
    (8, 8 * 2048 * 8 + 77, True, 0, False, "r%4", "3r+1"),
    (8, 8 * 2048 * 8 + 77, True, 0, True, "3r+1", None),
    (8, 8 * 2048 * 8 + 77, True, 2, False, "one-off", "r%4"),   # wire order
    (8, 99999, False, 0, False, "r%4", "r%4"),
    (8, 99999, False, 0, True, "3r+1", None),
    (3, 3 * 8192 * 2 + 5, True, 0, True, "r%4", None),          # IEEE divide, in place
    (16, 16 * 8192 + 9, True, 0, False, "3r+1", "r%4"),
    (64, 64 * 2048 + 9, True, 0, True, "r%4", None),            # chunks end inside tiles
    (64, 1000, True, 0, False, "r%4", "3r+1"),                  # C < tile: every tile straddles
    (64, 64 * 8192 * 3 + 1, True, 0, False, "3r+1", "r%4"),
    (4, 40, True, 0, False, "r%4", "3r+1"),                     # N below the lead
    (5, 5 * 4096 * 3 + 2, False, 0, True, "r%4", None),
]


@pytest.mark.parametrize("K,N,bf16,order,inplace,ipat,opat", AR_CASES)
def test_allreduce_ranks_in_mixed_phases(K, N, bf16, order, inplace, ipat, opat):
    import torch
    xs = make_inputs(K, N, bf16, K * 31 + N)
    ins = [Guarded(N, torch_dt(bf16), quad_phase(ipat, r), xs[r]) for r in range(K)]
    outs = ins if inplace else [Guarded(N, torch_dt(bf16), quad_phase(opat, r)) for r in range(K)]
    zr().zr_allreduce([g.ptr() for g in ins], [g.ptr() for g in outs], N, average=True, fused=True,
                      order=order, dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    want = oracle.allreduce(xs, N, average=True, wire=(order == 2))
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(want[r])), f"rank {r}"
        assert outs[r].guards_intact() and ins[r].guards_intact()


def free_bound_ok(got, exact, absum, K, out_bf16=False):
    ex = exact / K
    bound = 1e-5 * absum / K + (bf16_ulp(ex) if out_bf16 else 0)
    gotf = (oracle.bf16_to_f32(got) if out_bf16 else got).astype(np.float64)
    return bool(np.all(np.abs(gotf - ex) <= bound))


@pytest.mark.parametrize("K,N,bf16", [(8, 8 * 2048 * 4 + 77, True), (16, 50001, False),
                                      (64, 64 * 40000 + 7, True)])
def test_free_order_ranks_in_mixed_phases(K, N, bf16):
    # within the free order's bound of the exact sum
    import torch
    xs = make_inputs(K, N, bf16, 4242 + K)
    C = -(-N // K)
    ins = [Guarded(N, torch_dt(bf16), r % 4, xs[r]) for r in range(K)]
    outs = [Guarded(C, torch.float32, (r + 1) % 4) for r in range(K)]
    zr().zr_reduce_scatter_avg([g.ptr() for g in ins], N, [g.ptr() for g in outs], chunk_shift=1,
                               average=True, order=1, in_dtype=torch_dt(bf16), out_dtype=torch.float32)
    torch.cuda.synchronize()
    xf = np.stack([oracle.bf16_to_f32(x) if bf16 else x for x in xs])
    xp = np.zeros((K, K * C), dtype=np.float32)
    xp[:, :N] = xf
    exact, absum = oracle.exact_sum_points(xp)
    for q in range(K):
        j = (q + 1) % K
        ex = exact[j * C:(j + 1) * C] / K
        bound = 1e-5 * absum[j * C:(j + 1) * C] / K
        got = outs[q].get().astype(np.float64)
        assert np.all(np.abs(got - ex) <= bound), f"rank {q}"
        assert outs[q].guards_intact()


@pytest.mark.parametrize("ws", [False, True], ids=["args", "workspace"])
@pytest.mark.parametrize("K,sizes,bf16,shift", [
    (8, [8 * 8192 * 2 + 13, 999, 8 * 4096 + 7], True, 1),
    (8, [8 * 4096 * 3 + 1, 5, 77777], False, 0),
    (3, [3 * 8192 + 2, 1, 40000], True, 2),
    (64, [64 * 2048 + 63, 64 * 100], True, 1),
])
def test_all_gather_fulls_in_mixed_phases(K, sizes, bf16, shift, ws):
    # full buffer r at its own 16-byte phase, shard r at another
    import torch
    segs, soff, foff = [], 0, 0
    for n in sizes:
        segs.append((soff, foff, n))
        soff += -(-n // K) + 1
        foff += n + 3
    dt = np.uint16 if bf16 else np.float32
    per = 8 if bf16 else 4
    rng = np.random.default_rng(7 + K)
    shard_np = [(rng.integers(0, 65535, size=soff).astype(np.uint16) if bf16 else
                 rng.standard_normal(soff).astype(np.float32)) for _ in range(K)]
    shards = [Guarded(soff, torch_dt(bf16), (3 * r + 1) % per, shard_np[r]) for r in range(K)]
    fulls = [Guarded(foff, torch_dt(bf16), (5 * r) % per, np.zeros(foff, dtype=dt)) for r in range(K)]
    wsb = None
    if ws:
        wsb = torch.empty(max(256, zr().zr_workspace_bytes(K, len(segs))), dtype=torch.uint8, device="cuda")
    zr().zr_all_gather([g.ptr() for g in shards], [g.ptr() for g in fulls], segs, chunk_shift=shift,
                       dtype=torch_dt(bf16), workspace=wsb)
    torch.cuda.synchronize()
    want = [np.zeros(foff, dtype=dt) for _ in range(K)]
    oracle.all_gather(shard_np, want, segs, shift)
    for r in range(K):
        assert np.array_equal(bits(fulls[r].get()), bits(want[r])), f"rank {r}"
        assert fulls[r].guards_intact() and shards[r].guards_intact()


@pytest.mark.parametrize("K,N,bf16,inplace", [(8, 8 * 2048 * 8 + 77, True, False), (64, 64 * 2048 + 9, True, True),
                                              (5, 5 * 4096 * 3 + 2, False, True)])
def test_allreduce_free_order_ranks_in_mixed_phases(K, N, bf16, inplace):
    # every rank holds the same result, within the free order's bound
    import torch
    xs = make_inputs(K, N, bf16, 999 + K)
    ins = [Guarded(N, torch_dt(bf16), (3 * r + 1) % 4, xs[r]) for r in range(K)]
    outs = ins if inplace else [Guarded(N, torch_dt(bf16), r % 4) for r in range(K)]
    zr().zr_allreduce([g.ptr() for g in ins], [g.ptr() for g in outs], N, average=True, fused=True,
                      order=1, dtype=torch_dt(bf16))
    torch.cuda.synchronize()
    xf = np.stack([oracle.bf16_to_f32(x) if bf16 else x for x in xs])
    exact, absum = oracle.exact_sum_points(xf)
    first = outs[0].get()
    assert free_bound_ok(first, exact, absum, K, out_bf16=bf16)
    for r in range(K):
        assert np.array_equal(bits(outs[r].get()), bits(first)), f"rank {r}"
        assert outs[r].guards_intact()


def test_discrete_free_order_ranks_in_mixed_phases():
    import torch
    K, sizes = 16, [70001, 5, 300003]
    N = sum(sizes) + 11
    C = -(-N // K)
    frags_np = [[synth.host_normal_bf16(SEED + 9, r * 4096 + p, 0, n, 1.0, 0.01, 1e4)
                 for p, n in enumerate(sizes)] for r in range(K)]
    frags = [[Guarded(n, torch.bfloat16, (r + p) % 4, frags_np[r][p]) for p, n in enumerate(sizes)]
             for r in range(K)]
    outs = [Guarded(C, torch.float32, 1) for _ in range(K)]
    zr().zr_reduce_scatter_frags([[g.ptr() for g in row] for row in frags], sizes, N,
                                 [g.ptr() for g in outs], chunk_shift=1, average=True, order=1,
                                 in_dtype=torch.bfloat16, out_dtype=torch.float32)
    torch.cuda.synchronize()
    bucket = oracle.flatten(frags_np, sizes, N)
    xp = np.zeros((K, K * C), dtype=np.float32)
    xp[:, :N] = np.stack([oracle.bf16_to_f32(x) for x in bucket])
    exact, absum = oracle.exact_sum_points(xp)
    for q in range(K):
        j = (q + 1) % K
        assert free_bound_ok(outs[q].get(), exact[j * C:(j + 1) * C], absum[j * C:(j + 1) * C], K), f"rank {q}"
        assert outs[q].guards_intact()
