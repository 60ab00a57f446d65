"""Workspace-staged descriptor tables on the GPU.

A bucket of many fragments at K = 64 (256 pointers per argument block, so 4
fragments per launch) goes out as one launch when its table is staged in a
workspace, and as one launch per 4 fragments without it; both are bit-exact
against the oracle's flatten followed by its reduce-scatter ("DeepSpeed
ZeRO-3 源码解析", 3.1: one operation per bucket, not one per parameter; 5.2:
the reduce over the fragment list). Also: the staged table's size stays
within zr_workspace_bytes, calls on one stream may share a workspace, and a
workspace too small for the table leaves every output untouched.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import Guarded, bits

pytestmark = pytest.mark.gpu

SEED = 0x5A5200B0
K = 64


def zr():
    import gradient_sync_zr_amd as m
    return m


def fragments(K, F, seed, lo=1, hi=4000):
    """F fragments per rank with sizes uniform in [lo, hi), seeded values with
    outliers; on the device they are views into one buffer per rank, each
    fragment 0-7 elements after the previous one (so their quad phases
    vary), like the gradients of one module's parameters."""
    rng = np.random.default_rng(seed)
    sizes = [int(x) for x in rng.integers(lo, hi, size=F)]
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
        host = np.full(o, 0xFFFF, dtype=np.uint16)
        for p, n in enumerate(sizes):
            host[offs[p]:offs[p] + n] = frags_np[r][p]
        g = Guarded(o, torch_bf16(), 0, host)
        bufs.append(g)
        ptrs.append([g.ptr() + 2 * offs[p] for p in range(F)])
    return sizes, frags_np, ptrs, bufs


def torch_bf16():
    import torch
    return torch.bfloat16


def test_k64_many_fragments_one_launch_with_workspace():
    import torch
    F = 300
    sizes, frags_np, fp, bufs = fragments(K, F, 1)
    N = -(-sum(sizes) // K) * K + K * 3
    C = N // K
    need = zr().zr_workspace_bytes(K, F)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    bucket = oracle.flatten(frags_np, sizes, N)
    want = oracle.reduce_scatter(bucket, N, np.float32, shift=1, average=True)

    with_ws = [Guarded(C, torch.float32, 0) for _ in range(K)]
    without = [Guarded(C, torch.float32, 0) for _ in range(K)]
    one_shot = [Guarded(C, torch.float32, 0) for _ in range(K)]
    dts = dict(in_dtype=torch.bfloat16, out_dtype=torch.float32)
    p_ws = zr().RsfPlan(fp, sizes, N, [g.ptr() for g in with_ws], workspace=ws, **dts)
    p_args = zr().RsfPlan(fp, sizes, N, [g.ptr() for g in without], **dts)
    info_ws, info_args = p_ws.info(), p_args.info()
    print(f"K={K} F={F}: {info_args['launches']} launches without a workspace, "
          f"{info_ws['launches']} with {info_ws['table_bytes']} staged bytes", flush=True)
    assert info_ws["launches"] == 1
    assert info_args["launches"] == -(-F // 4) >= 64
    assert 0 < info_ws["table_bytes"] <= need
    p_ws.launch()
    p_args.launch()
    ws2 = torch.empty(need, dtype=torch.uint8, device="cuda")
    zr().zr_reduce_scatter_frags(fp, sizes, N, [g.ptr() for g in one_shot], workspace=ws2, **dts)
    torch.cuda.synchronize()
    for q in range(K):
        for res in (with_ws, without, one_shot):
            assert np.array_equal(bits(res[q].get()), bits(want[q])), f"rank {q}"
            assert res[q].guards_intact()
    # the plan launches again from the same staged table
    for g in with_ws:
        g.t.zero_()
    p_ws.launch()
    torch.cuda.synchronize()
    for q in range(K):
        assert np.array_equal(bits(with_ws[q].get()), bits(want[q]))
    p_ws.close()
    p_args.close()


def test_k64_flatten_plan_one_launch_with_workspace():
    import torch
    F = 260
    sizes, frags_np, fp, bufs = fragments(K, F, 2)
    padded = -(-sum(sizes) // K) * K
    ws = torch.empty(zr().zr_workspace_bytes(K, F), dtype=torch.uint8, device="cuda")
    a = [Guarded(padded, torch.bfloat16, 0, np.full(padded, 0x3F80, dtype=np.uint16)) for _ in range(K)]
    b = [Guarded(padded, torch.bfloat16, 0, np.full(padded, 0x3F80, dtype=np.uint16)) for _ in range(K)]
    p_ws = zr().FlatPlan(fp, sizes, [g.ptr() for g in a], padded, dtype=torch.bfloat16, workspace=ws)
    p_args = zr().FlatPlan(fp, sizes, [g.ptr() for g in b], padded, dtype=torch.bfloat16)
    assert p_ws.info()["launches"] == 1
    assert p_args.info()["launches"] == -(-F // 4)
    p_ws.launch()
    p_args.launch()
    torch.cuda.synchronize()
    want = oracle.flatten(frags_np, sizes, padded)
    for r in range(K):
        assert np.array_equal(bits(a[r].get()), bits(want[r])), f"rank {r}"
        assert np.array_equal(bits(b[r].get()), bits(want[r])), f"rank {r}"
        assert a[r].guards_intact() and b[r].guards_intact() and bufs[r].guards_intact()
    p_ws.close()
    p_args.close()


def test_calls_on_one_stream_share_a_workspace():
    # the second call's table is copied after the first call's kernel has
    # read its own (stream order), so one workspace serves both
    import torch
    K8, F = 8, 70
    ws = torch.empty(zr().zr_workspace_bytes(K8, F + 9), dtype=torch.uint8, device="cuda")
    results = []
    for n_frag, seed in ((F, 3), (F + 9, 4)):
        sizes, frags_np, fp, bufs = fragments(K8, n_frag, seed)
        N = -(-sum(sizes) // K8) * K8
        outs = [Guarded(N // K8, torch.float32, 0) for _ in range(K8)]
        zr().zr_reduce_scatter_frags(fp, sizes, N, [g.ptr() for g in outs], workspace=ws,
                                     in_dtype=torch.bfloat16, out_dtype=torch.float32)
        results.append((sizes, frags_np, N, outs, bufs))
    torch.cuda.synchronize()
    for sizes, frags_np, N, outs, _ in results:
        want = oracle.reduce_scatter(oracle.flatten(frags_np, sizes, N), N, np.float32, shift=1,
                                     average=True)
        for q in range(K8):
            assert np.array_equal(bits(outs[q].get()), bits(want[q])), f"rank {q}"


def test_workspace_too_small_writes_nothing():
    import torch
    F = 40
    sizes, frags_np, fp, bufs = fragments(K, F, 5)
    N = -(-sum(sizes) // K) * K
    init = np.full(N // K, 7.0, dtype=np.float32)
    outs = [Guarded(N // K, torch.float32, 0, init) for _ in range(K)]
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(zr().ZrError) as e:
        zr().zr_reduce_scatter_frags(fp, sizes, N, [g.ptr() for g in outs], workspace=ws,
                                     in_dtype=torch.bfloat16, out_dtype=torch.float32)
    assert e.value.status == zr().ZR_ERR_WORKSPACE
    torch.cuda.synchronize()
    for q in range(K):
        assert np.array_equal(outs[q].get(), init)
