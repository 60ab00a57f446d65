"""The hot path captured in a HIP graph.

The library's calls allocate nothing, issue no memset and never synchronise
the device, so a caller can capture them. One graph holds a reduce-scatter,
an accumulating reduce-scatter, a discrete reduce-scatter (the one-shot call
and a prepared plan), a bucket flatten, a fused and a composed all-reduce
(out of place), an all-gather and a prepared reduce-scatter plan; and, for a bucket of more fragments than
one argument block holds, a discrete plan and a flatten plan whose tables
were staged in workspaces at creation (one launch each), and a one-shot
discrete call given a workspace, which under capture goes out as argument
launches rather than record a copy from host memory. It is replayed several times; before
each replay the program rewrites the inputs eagerly and synchronises, and
after it every output is compared bit for bit with the same calls made
eagerly on the same inputs.
"""
import numpy as np
import pytest

import synth
from gpu_util import bits

pytestmark = pytest.mark.gpu

K = 8
N = K * 4096 * 3 + 40
SIZES = [5000, 37, 12288, 4096 * 3 + 17]
MANY = [1 + 301 * i for i in range(40)]  # more fragments than one argument block holds at K = 8
SEED = 0x5A5200C0


def test_graph_replays_match_eager_calls():
    import torch
    import gradient_sync_zr_amd as zr
    C = -(-N // K)
    F = sum(SIZES)
    NF = -(-F // K) * K
    CF = NF // K
    x = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in SIZES] for _ in range(K)]
    many = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in MANY] for _ in range(K)]
    NM = -(-sum(MANY) // K) * K
    shards = [torch.empty(C, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    segs = [(0, 0, N)]

    def outputs():
        return dict(rs=[torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)],
                    rsplan=[torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)],
                    acc=[torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)],
                    frag=[torch.empty(CF, dtype=torch.float32, device="cuda") for _ in range(K)],
                    plan=[torch.empty(CF, dtype=torch.float32, device="cuda") for _ in range(K)],
                    flat=[torch.empty(NF, dtype=torch.bfloat16, device="cuda") for _ in range(K)],
                    ar=[torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)],
                    arc=[torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)],
                    scratch=torch.empty(K * C, dtype=torch.bfloat16, device="cuda"),
                    ag=[torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)],
                    wsplan=[torch.empty(NM // K, dtype=torch.float32, device="cuda") for _ in range(K)],
                    wscall=[torch.empty(NM // K, dtype=torch.float32, device="cuda") for _ in range(K)],
                    wsflat=[torch.empty(NM, dtype=torch.bfloat16, device="cuda") for _ in range(K)])

    def ws():
        return torch.empty(zr.zr_workspace_bytes(K, len(MANY)), dtype=torch.uint8, device="cuda")

    g_out, e_out = outputs(), outputs()
    g_rsplan = zr.RsPlan(x, N, g_out["rsplan"], chunk_shift=1, average=True)
    e_rsplan = zr.RsPlan(x, N, e_out["rsplan"], chunk_shift=1, average=True)
    g_plan = zr.RsfPlan(frags, SIZES, NF, g_out["plan"], chunk_shift=1, average=True)
    e_plan = zr.RsfPlan(frags, SIZES, NF, e_out["plan"], chunk_shift=1, average=True)
    g_wsplan = zr.RsfPlan(many, MANY, NM, g_out["wsplan"], workspace=ws())
    e_wsplan = zr.RsfPlan(many, MANY, NM, e_out["wsplan"], workspace=ws())
    g_wsflat = zr.FlatPlan(many, MANY, g_out["wsflat"], NM, workspace=ws())
    e_wsflat = zr.FlatPlan(many, MANY, e_out["wsflat"], NM, workspace=ws())
    assert g_wsplan.info()["launches"] == 1 and g_wsflat.info()["launches"] == 1
    g_ws, e_ws = ws(), ws()

    def work(o, plan, wsplan, wsflat, wsbuf, rsplan):
        zr.zr_reduce_scatter_avg(x, N, o["rs"], chunk_shift=1, average=True)
        rsplan.launch()
        zr.zr_reduce_scatter_avg(x, N, o["acc"], chunk_shift=1, average=True, accumulate=True)
        zr.zr_reduce_scatter_frags(frags, SIZES, NF, o["frag"], chunk_shift=1, average=True)
        plan.launch()
        zr.zr_flatten_bucket(frags, SIZES, o["flat"], NF)
        zr.zr_allreduce(x, o["ar"], N, average=False, fused=True)
        zr.zr_allreduce(x, o["arc"], N, average=True, fused=False, scratch=o["scratch"])
        zr.zr_all_gather(shards, o["ag"], segs, chunk_shift=0)
        wsplan.launch()
        wsflat.launch()
        zr.zr_reduce_scatter_frags(many, MANY, NM, o["wscall"], workspace=wsbuf)

    def fill(tag):
        for r in range(K):
            synth.dev_normal_bf16(x[r], SEED + tag, r, 0, 1.0)
            synth.dev_normal_bf16(shards[r], SEED + tag, 100 + r, 0, 1.0)
            for p in range(len(SIZES)):
                synth.dev_normal_bf16(frags[r][p], SEED + tag, 200 + 8 * r + p, 0, 1.0)
            for p in range(len(MANY)):
                synth.dev_normal_bf16(many[r][p], SEED + tag, 300 + 64 * r + p, 0, 1.0)
        for o in (g_out, e_out):
            for r in range(K):
                o["acc"][r].fill_(0.5 * (tag + 1))
        torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(g_out, g_plan, g_wsplan, g_wsflat, g_ws, g_rsplan)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        work(g_out, g_plan, g_wsplan, g_wsflat, g_ws, g_rsplan)
    torch.cuda.synchronize()
    for tag in (1, 2, 3):
        fill(tag)
        graph.replay()
        torch.cuda.synchronize()
        work(e_out, e_plan, e_wsplan, e_wsflat, e_ws, e_rsplan)
        torch.cuda.synchronize()
        for key in ("rs", "rsplan", "acc", "frag", "plan", "flat", "ar", "arc", "ag", "wsplan",
                    "wscall", "wsflat"):
            for r in range(K):
                got = g_out[key][r].cpu()
                want = e_out[key][r].cpu()
                if got.dtype == torch.bfloat16:
                    got, want = got.view(torch.int16), want.view(torch.int16)
                assert np.array_equal(bits(got.numpy()), bits(want.numpy())), (tag, key, r)
    for p in (g_plan, e_plan, g_wsplan, e_wsplan, g_wsflat, e_wsflat, g_rsplan, e_rsplan):
        p.close()
