"""Concurrent callers: the library keeps no mutable state between calls.

Four host threads each own a stream and their own buffers. Every thread issues, ten times over, a
reduce-scatter, a discrete reduce-scatter, a fused out-of-place all-reduce and an all-gather on its
stream; ctypes releases the GIL during each call, so the calls enter the library together. After every
round each thread checks its outputs bit for bit against the oracle, which was computed before the
threads started.

A fifth thread makes invalid calls at the same time. Each of its calls must fail with that call's own
message. The error text is per thread, so the valid callers never see it.
"""
import threading

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bits, down16, up16

pytestmark = pytest.mark.gpu

K = 8
N = K * 40000 + 13
SIZES = [3, 20000, 7, 31000]
THREADS = 4
ROUNDS = 10


def test_concurrent_callers_get_their_own_results():
    import torch
    import gradient_sync_zr_amd as zr
    C = -(-N // K)
    F = sum(SIZES)
    NF = F + 5
    CF = -(-NF // K)
    cuts = np.cumsum([0] + SIZES)
    work = []
    for t in range(THREADS):
        xs = [synth.host_normal_bf16(0x5A5200D0 + t, r, 0, N, 1.0, 0.01, 1e4) for r in range(K)]
        fl = [synth.host_normal_bf16(0x5A5200E0 + t, r, 0, F, 1.0) for r in range(K)]
        frags_np = [[fl[r][cuts[p]:cuts[p + 1]].copy() for p in range(len(SIZES))] for r in range(K)]
        w = dict(
            x=[up16(a) for a in xs],
            frags=[[up16(f) for f in row] for row in frags_np],
            shards=[up16(a[:C]) for a in xs],
            rs=[torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)],
            rsf=[torch.empty(CF, dtype=torch.float32, device="cuda") for _ in range(K)],
            ar=[torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)],
            ag=[torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)],
            want_rs=oracle.reduce_scatter(xs, N, np.float32, shift=1, average=True),
            want_rsf=oracle.reduce_scatter(oracle.flatten(frags_np, SIZES, NF), NF, np.float32,
                                           shift=1, average=True),
            want_ar=oracle.allreduce(xs, N)[0],
            want_ag=[np.zeros(N, dtype=np.uint16) for _ in range(K)],
            stream=torch.cuda.Stream(),
        )
        oracle.all_gather([a[:C] for a in xs], w["want_ag"], [(0, 0, N)], 0)
        work.append(w)
    torch.cuda.synchronize()
    failures = []
    start = threading.Barrier(THREADS + 1)

    def caller(w):
        try:
            start.wait()
            with torch.cuda.stream(w["stream"]):
                for i in range(ROUNDS):
                    for o in w["rs"] + w["rsf"]:
                        o.fill_(float("nan"))
                    for o in w["ar"] + w["ag"]:
                        o.view(torch.int16).fill_(-1)
                    zr.zr_reduce_scatter_avg(w["x"], N, w["rs"], chunk_shift=1, average=True)
                    zr.zr_reduce_scatter_frags(w["frags"], SIZES, NF, w["rsf"], chunk_shift=1,
                                               average=True)
                    zr.zr_allreduce(w["x"], w["ar"], N)
                    zr.zr_all_gather(w["shards"], w["ag"], [(0, 0, N)], chunk_shift=0)
                    w["stream"].synchronize()
                    for r in range(K):
                        assert np.array_equal(bits(w["rs"][r].cpu().numpy()), bits(w["want_rs"][r]))
                        assert np.array_equal(bits(w["rsf"][r].cpu().numpy()),
                                              bits(w["want_rsf"][r]))
                        assert np.array_equal(down16(w["ar"][r]), w["want_ar"])
                        assert np.array_equal(down16(w["ag"][r]), w["want_ag"][r])
                    assert zr.zr_last_error() == ""
        except Exception as e:  # reported by the main thread
            failures.append(repr(e))

    def bad_caller():
        try:
            start.wait()
            for i in range(200):
                for K_bad, what in ((0, "K=0"), (65, "K=65")):
                    try:
                        zr.zr_reduce_scatter_avg([0] * K_bad, 16, [0] * K_bad,
                                                 in_dtype=torch.bfloat16, out_dtype=torch.float32)
                    except zr.ZrError as e:
                        assert what in str(e), (what, str(e))
                    else:
                        raise AssertionError(f"{what} was accepted")
        except Exception as e:
            failures.append(repr(e))

    threads = [threading.Thread(target=caller, args=(w,)) for w in work]
    threads.append(threading.Thread(target=bad_caller))
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=300)
        assert not th.is_alive(), "a caller did not finish"
    assert not failures, failures
