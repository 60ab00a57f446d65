"""The scheduler on the GPU, with forced delays.

A bounded delay kernel (tests/kit/testkit.hip) holds a stream busy so that a
missing wait would let a later write overtake the reduction. Checks follow the
validation list of "ZeRO-1/2 average_tensor serializes backward compute
behind the preceding reduction" (DeepSpeed issue 8364): the ping-pong reuse
race, the multi-producer race, and that compute producing the next bucket
does not stop while the previous reduction is still running. Results are
checked bit for bit against the oracle.
"""
import ctypes
import os
import time

import numpy as np
import pytest

import oracle
import synth
from conftest import ROOT
from gpu_util import bits, up16

pytestmark = pytest.mark.gpu

K, N = 8, 8 * 2048 * 16 + 40
SEED = 0x5A5200B0

_kit = None


def kit():
    global _kit
    if _kit is None:
        L = ctypes.CDLL(os.path.join(ROOT, "tests", "kit", "libtestkit.so"))
        L.tk_delay.argtypes = [ctypes.c_longlong, ctypes.c_longlong, ctypes.c_void_p,
                               ctypes.c_void_p]
        L.tk_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int)]
        _kit = L
    return _kit


def delay(ms, stream):
    khz = ctypes.c_int(0)
    assert kit().tk_clock_khz(ctypes.byref(khz)) == 0 and khz.value > 0
    ticks = int(ms * khz.value)
    assert kit().tk_delay(ticks, 50_000_000, None, stream.cuda_stream) == 0


def host_bucket(tag):
    return [synth.host_normal_bf16(SEED + tag, r, 0, N, 1.0, 0.01, 1e4) for r in range(K)]


def expected(xs):
    return oracle.reduce_scatter(xs, N, np.float32, shift=1, average=True)


_streams = {}


def streams():
    """The same reduction and producer streams for every test in this module:
    the runtime spreads streams over a few hardware queues, and streams that
    end up sharing a queue cannot overlap, so the module keeps to two."""
    import torch
    if not _streams:
        _streams["red"] = torch.cuda.Stream()
        _streams["prod"] = torch.cuda.Stream()
        _streams["prod2"] = torch.cuda.Stream()
    return _streams["red"], _streams["prod"]


def setup():
    import torch
    import gradient_sync_zr_amd as zr
    red, prod = streams()
    C = -(-N // K)
    bufs = [[torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
            for _ in range(2)]
    outs = [[torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
            for _ in range(3)]
    sched = zr.Sched(n_buffers=2, max_producers=2, reduction_stream=red)
    return torch, red, prod, bufs, outs, sched


def write(torch, stream, dst_list, host_list):
    src = [up16(h) for h in host_list]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for d, s in zip(dst_list, src):
            d.copy_(s)
    return src


def test_pingpong_reuse_waits_for_the_reduction():
    torch, red, prod, bufs, outs, sched = setup()
    A, B = host_bucket(1), host_bucket(2)
    sched.acquire(0, prod)
    keep = write(torch, prod, bufs[0], A)
    delay(300, red)                         # the reduction of bucket A starts late
    sched.submit_rs(0, [prod], bufs[0], N, outs[0])
    sched.acquire(0, prod)                  # reuse: must wait for that reduction
    keep += write(torch, prod, bufs[0], B)
    sched.submit_rs(0, [prod], bufs[0], N, outs[1])
    sched.flush(prod)
    torch.cuda.synchronize()
    for q, (wa, wb) in enumerate(zip(expected(A), expected(B))):
        assert np.array_equal(bits(outs[0][q].cpu().numpy()), bits(wa)), f"bucket A rank {q}"
        assert np.array_equal(bits(outs[1][q].cpu().numpy()), bits(wb)), f"bucket B rank {q}"
    sched.close()


def streams_overlap(torch, red, prod):
    """Whether work on `prod` can finish while `red` is busy at all."""
    x = torch.zeros(1024, device="cuda")
    torch.cuda.synchronize()
    delay(400, red)
    r = torch.cuda.Event()
    r.record(red)
    with torch.cuda.stream(prod):
        x.add_(1)
    p = torch.cuda.Event()
    p.record(prod)
    t0 = time.time()
    while not p.query() and time.time() - t0 < 0.3:
        time.sleep(0.002)
    ok = p.query() and not r.query()
    torch.cuda.synchronize()
    return ok


def test_next_bucket_not_blocked_by_previous_reduction():
    torch, red, prod, bufs, outs, sched = setup()
    if not streams_overlap(torch, red, prod):
        sched.close()
        pytest.skip("the runtime runs these two streams on one hardware queue, so no "
                    "overlap can be observed")
    A, B = host_bucket(3), host_bucket(4)
    srcA = [up16(h) for h in A]
    srcB = [up16(h) for h in B]
    torch.cuda.synchronize()
    sched.acquire(0, prod)
    with torch.cuda.stream(prod):
        for d, s in zip(bufs[0], srcA):
            d.copy_(s)
    delay(1500, red)                        # bucket 0's reduction is held for 1.5 s
    sched.submit_rs(0, [prod], bufs[0], N, outs[0])
    red_done = torch.cuda.Event()
    red_done.record(red)
    sched.acquire(1, prod)                  # the other buffer: no wait on bucket 0
    with torch.cuda.stream(prod):
        for d, s in zip(bufs[1], srcB):
            d.copy_(s)
    prod_done = torch.cuda.Event()
    prod_done.record(prod)
    t0 = time.time()
    while not prod_done.query() and time.time() - t0 < 1.0:
        time.sleep(0.002)
    assert prod_done.query(), "producer of bucket 1 was held behind bucket 0's reduction"
    assert not red_done.query(), "the forced delay ended too early to show the overlap"
    sched.submit_rs(1, [prod], bufs[1], N, outs[1])
    sched.flush(prod)
    torch.cuda.synchronize()
    for q, (wa, wb) in enumerate(zip(expected(A), expected(B))):
        assert np.array_equal(bits(outs[0][q].cpu().numpy()), bits(wa))
        assert np.array_equal(bits(outs[1][q].cpu().numpy()), bits(wb))
    sched.close()


def test_multi_producer_reduction_waits_for_every_producer():
    torch, red, prod, bufs, outs, sched = setup()
    prod2 = _streams["prod2"]
    A = host_bucket(5)
    src = [up16(h) for h in A]
    torch.cuda.synchronize()
    sched.acquire(0, prod)
    half = K // 2
    with torch.cuda.stream(prod):
        for r in range(half):
            bufs[0][r].copy_(src[r])
    delay(300, prod2)                       # the second producer is late
    with torch.cuda.stream(prod2):
        for r in range(half, K):
            bufs[0][r].copy_(src[r])
    sched.submit_rs(0, [prod, prod2], bufs[0], N, outs[0])
    sched.flush(prod)
    torch.cuda.synchronize()
    for q, w in enumerate(expected(A)):
        assert np.array_equal(bits(outs[0][q].cpu().numpy()), bits(w)), f"rank {q}"
    sched.close()


def test_rapid_reuse_and_flush_match_serial_results():
    # gradients and results with overlap on equal those of a plain serial run
    torch, red, prod, bufs, outs, sched = setup()
    import gradient_sync_zr_amd as zr
    tags = list(range(10, 16))
    hosts = {t: host_bucket(t) for t in tags}
    srcs = {t: [up16(h) for h in hosts[t]] for t in tags}
    C = -(-N // K)
    res = {t: [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)] for t in tags}
    torch.cuda.synchronize()
    for i, t in enumerate(tags):
        b = i % 2
        sched.acquire(b, prod)
        with torch.cuda.stream(prod):
            for d, s in zip(bufs[b], srcs[t]):
                d.copy_(s)
        sched.submit_rs(b, [prod], bufs[b], N, res[t])
    sched.flush(prod)
    torch.cuda.synchronize()
    for t in tags:
        serial = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
        zr.zr_reduce_scatter_avg(srcs[t], N, serial, chunk_shift=1, average=True)
        torch.cuda.synchronize()
        for q in range(K):
            assert torch.equal(res[t][q].view(torch.int32), serial[q].view(torch.int32))
    sched.close()


def test_zero2_sync_reduces_what_the_producer_wrote():
    # the backward pass, through Zero2GradSync's produce hook, writes each
    # bucket's gradients on the producer stream after a delay: a reduction
    # that did not wait for its producer would reduce the zeros left there
    import torch
    from gradient_sync_zr_amd.steps import Zero2GradSync
    red, prod = streams()
    bucket = 8 * 4096 + 5
    total = 3 * bucket + 1234
    grads = [torch.zeros(total, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    P = sum(-(-min(bucket, total - s) // K) for s in range(0, total, bucket))
    parts = [torch.empty(P, dtype=torch.float32, device="cuda") for _ in range(K)]
    sync = Zero2GradSync(grads, parts, bucket, chunk_shift=1, average=True, reduction_stream=red)
    seen = []

    def produce(i, stream):
        n, _, _, start, _ = sync.buckets[i]
        seen.append(i)
        delay(20, stream)
        for r in range(K):
            synth.dev_normal_bf16(grads[r][start:start + n], SEED + 9, r, start, 1.0, stream=stream)

    sync.step(producer_stream=prod, produce=produce)
    torch.cuda.synchronize()
    assert seen == list(range(len(sync.buckets)))
    for n, _, _, start, poff in sync.buckets:
        xs = [synth.host_normal_bf16(SEED + 9, r, start, n, 1.0) for r in range(K)]
        want = oracle.reduce_scatter(xs, n, np.float32, shift=1, average=True)
        C = -(-n // K)
        for q in range(K):
            got = parts[q][poff:poff + C].cpu().numpy()
            assert np.array_equal(bits(got), bits(want[q])), f"bucket at {start}, rank {q}"
    sync.close()


def test_scheduler_errors_on_gpu():
    torch, red, prod, bufs, outs, sched = setup()
    import gradient_sync_zr_amd as zr
    with pytest.raises(zr.ZrError):
        sched.submit_rs(0, [prod], bufs[0], N, outs[0])   # not acquired
    sched.acquire(1, prod)
    with pytest.raises(zr.ZrError):
        sched.acquire(1, prod)
    with pytest.raises(zr.ZrError):
        sched.submit_rs(1, [prod, prod, prod], bufs[1], N, outs[0])  # > max_producers
    with pytest.raises(zr.ZrError):
        sched.submit_rs(1, [prod], bufs[1], N, [bufs[1][0]] * K)     # aliasing outputs
    sched.close()
