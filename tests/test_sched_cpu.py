"""Scheduler logic on the CPU.

The scheduler core that libzr uses is compiled here against a backend that
only logs (tests/kit/sched_sim.cpp). Each test plays a host program (producer
writes, acquire, submit, flush), turns the log into per-stream operations and
replays them on a discrete-event model with stream/event semantics: a wait
refers to the event's most recent record at the time the wait was issued.

What is checked follows the validation list of "ZeRO-1/2 average_tensor
serializes backward compute behind the preceding reduction" (DeepSpeed issue
8364): the ping-pong reuse race, the multi-producer race, rapid reuse of both
buffer indices, and that compute producing bucket N+1 is not held behind
bucket N's reduction.
"""
import ctypes
import os

import numpy as np
import pytest

from conftest import ROOT

KIT = os.path.join(ROOT, "tests", "kit")
CREATE, DESTROY, RECORD, WAIT, LAUNCH = 1, 2, 3, 4, 5
OK, BAD_BUF, BAD_STATE, TOO_MANY, BACKEND, BAD_ARG = range(6)

_lib = None


def lib():
    global _lib
    if _lib is None:
        # SCHED_SIM_LIBRARY may name another build of the same simulator (the sanitizer
        # test runs this module against one)
        path = os.environ.get("SCHED_SIM_LIBRARY") or os.path.join(KIT, "libsched_sim.so")
        if not os.path.exists(path):
            import sys
            sys.path.insert(0, os.path.join(ROOT, "tests"))
            from kit import _build
            _build.build()
        L = ctypes.CDLL(path)
        L.sim_create.restype = ctypes.c_void_p
        L.sim_create.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_int)]
        for f in ("sim_acquire", "sim_flush"):
            getattr(L, f).argtypes = [ctypes.c_void_p, ctypes.c_int] + (
                [ctypes.c_int] if f == "sim_acquire" else [])
        L.sim_submit.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                 ctypes.c_int, ctypes.c_int]
        L.sim_log_size.restype = ctypes.c_int64
        L.sim_log_size.argtypes = [ctypes.c_void_p]
        L.sim_log.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.sim_destroy.argtypes = [ctypes.c_void_p]
        _lib = L
    return _lib


RED = 100  # reduction stream id


class Program:
    """Host program + replay. Streams are ints; work items have durations."""

    def __init__(self, n_buffers=2, max_prod=4, fail_on_call=-1):
        err = ctypes.c_int(-1)
        self.h = lib().sim_create(n_buffers, max_prod, RED, fail_on_call, ctypes.byref(err))
        self.init_err = err.value
        self.streams = {}
        self.seen = 0
        self.version = {}   # event id -> latest version (id, n)
        self.work = []      # (label, stream, index in that stream)
        self.waits = []     # (stream, event) of every wait the scheduler enqueued
        self.records = []   # (event, stream) of every record

    def close(self):
        lib().sim_destroy(self.h)

    def _q(self, s):
        return self.streams.setdefault(s, [])

    def _drain_log(self):
        n = lib().sim_log_size(self.h)
        buf = np.zeros(n, dtype=np.int64)
        if n:
            lib().sim_log(self.h, buf.ctypes.data)
        for i in range(self.seen, n, 3):
            op, a, b = (int(x) for x in buf[i:i + 3])
            if op == RECORD:
                self.records.append((a, b))
                v = self.version.get(a, 0) + 1
                self.version[a] = v
                self._q(b).append(("record", (a, v)))
            elif op == WAIT:
                self.waits.append((a, b))
                v = self.version.get(b, 0)
                if v:
                    self._q(a).append(("wait", (b, v)))
            elif op == LAUNCH:
                self.add_work(b, f"reduce{a}", self.red_time)
        self.seen = n

    red_time = 10.0

    def add_work(self, stream, label, dur):
        q = self._q(stream)
        q.append(("work", (label, dur)))
        self.work.append((label, stream, len(q) - 1))

    # host calls
    def write(self, producer, buf, dur=1.0):
        self.add_work(producer, f"write{buf}", dur)

    def acquire(self, buf, producer):
        st = lib().sim_acquire(self.h, buf, producer)
        self._drain_log()
        return st

    def submit(self, buf, producers, launch_ok=1):
        arr = (ctypes.c_int * max(1, len(producers)))(*producers)
        st = lib().sim_submit(self.h, buf, arr, len(producers), launch_ok)
        self._drain_log()
        return st

    def flush(self, caller):
        st = lib().sim_flush(self.h, caller)
        self._drain_log()
        return st

    def replay(self):
        """Returns {(stream, index): (start, end)} for work items."""
        pos = {s: 0 for s in self.streams}
        t = {s: 0.0 for s in self.streams}
        done_at = {}
        spans = {}
        progress = True
        while progress:
            progress = False
            for s, q in self.streams.items():
                while pos[s] < len(q):
                    kind, arg = q[pos[s]]
                    if kind == "work":
                        spans[(s, pos[s])] = (t[s], t[s] + arg[1])
                        t[s] += arg[1]
                    elif kind == "record":
                        done_at[arg] = t[s]
                    elif kind == "wait":
                        if arg not in done_at:
                            break
                        t[s] = max(t[s], done_at[arg])
                    pos[s] += 1
                    progress = True
        assert all(pos[s] == len(q) for s, q in self.streams.items()), "deadlock"
        return spans

    def spans_of(self, label):
        sp = self.replay()
        return [sp[(s, i)] for (lab, s, i) in self.work if lab == label]


def test_init_creates_events_and_reports_backend_failure():
    p = Program()
    assert p.init_err == OK
    p.close()
    p = Program(fail_on_call=3)
    assert p.init_err == BACKEND
    p.close()
    p = Program(n_buffers=0)
    assert p.init_err == BAD_ARG
    p.close()


def test_state_errors():
    p = Program(n_buffers=2, max_prod=2)
    assert p.submit(0, [1]) == BAD_STATE            # submit without acquire
    assert p.acquire(2, 1) == BAD_BUF
    assert p.acquire(-1, 1) == BAD_BUF
    assert p.acquire(0, 1) == OK
    assert p.acquire(0, 1) == BAD_STATE             # acquire twice
    assert p.submit(0, [1, 2, 3]) == TOO_MANY
    assert p.submit(0, [1], launch_ok=0) == BACKEND
    assert p.submit(0, [1]) == OK
    assert p.submit(0, [1]) == BAD_STATE            # double submit
    p.close()


def test_pingpong_reuse_waits_for_that_buffer_only():
    # producer 1 fills buffers 0,1,0,1,... ; reduction of each takes 10 units,
    # each write 1 unit. Reuse of buffer b must wait for b's last reduction.
    p = Program()
    prod = 1
    order = [0, 1, 0, 1, 0, 1]
    for b in order:
        assert p.acquire(b, prod) == OK
        p.write(prod, b)
        assert p.submit(b, [prod]) == OK
    assert p.flush(prod) == OK
    p.write(prod, "after")
    sp = p.replay()
    writes = {}
    reds = {}
    for (lab, s, i) in p.work:
        if lab.startswith("write"):
            writes.setdefault(lab, []).append(sp[(s, i)])
        if lab.startswith("reduce"):
            reds.setdefault(lab, []).append(sp[(s, i)])
    for b in (0, 1):
        w, r = writes[f"write{b}"], reds[f"reduce{b}"]
        for k in range(len(r)):
            assert r[k][0] >= w[k][1]          # reduction reads a finished bucket
            if k + 1 < len(w):
                assert w[k + 1][0] >= r[k][1]  # no overwrite while it is being read
    # the first write of buffer 1 is not held behind reduction 0
    assert writes["write1"][0][0] == writes["write0"][0][1]
    # after flush the caller's next work starts once every reduction ended
    end_all = max(e for v in reds.values() for (_, e) in v)
    assert writes["writeafter"][0][0] >= end_all


def test_compute_not_stalled_by_previous_bucket():
    # issue 8364's timeline: bucket N launches, compute prepares bucket N+1.
    # With per-buffer events the producer only waits when it reuses a buffer,
    # so with 2 buffers and 1-unit writes the producer runs ahead until the
    # third bucket.
    p = Program()
    prod = 1
    for b in (0, 1):
        p.acquire(b, prod)
        p.write(prod, b)
        p.submit(b, [prod])
    w = p.spans_of("write1")[0]
    r0 = p.spans_of("reduce0")[0]
    assert w[0] < r0[1]           # bucket 1 was written while bucket 0 was reducing


def test_multi_producer_reduction_waits_for_all():
    p = Program(max_prod=3)
    for b in (0, 1, 0):
        p.acquire(b, 1)
        p.write(1, b, dur=1.0)
        p.write(2, b, dur=5.0)   # a slower second producer of the same bucket
        p.write(3, b, dur=2.0)
        assert p.submit(b, [1, 2, 3]) == OK
    sp = p.replay()
    ends = {}
    for (lab, s, i) in p.work:
        ends.setdefault(lab, []).append((s, sp[(s, i)]))
    # first reduction of buffer 0 starts after all three producers' writes
    first_writes = [span for (s, span) in ends["write0"][:3]]
    r0 = [span for (s, span) in ends["reduce0"]][0]
    assert r0[0] >= max(e for (_, e) in first_writes)
    # missing a producer would break this: drop producer 2 and see the race
    q = Program(max_prod=3)
    q.acquire(0, 1)
    q.write(1, 0)
    q.write(2, 0, dur=5.0)
    q.submit(0, [1])
    sp = q.replay()
    r = q.spans_of("reduce0")[0]
    slow = [sp[(s, i)] for (lab, s, i) in q.work if lab == "write0" and s == 2][0]
    assert r[0] < slow[1]


def test_rapid_reuse_of_both_indices():
    p = Program()
    for _ in range(20):
        for b in (0, 1):
            assert p.acquire(b, 1) == OK
            p.write(1, b, dur=0.1)
            assert p.submit(b, [1]) == OK
    p.flush(1)
    sp = p.replay()
    items = sorted((sp[(s, i)], lab) for (lab, s, i) in p.work)
    # every buffer's write/reduce alternate without overlap
    for b in (0, 1):
        seq = [(span, lab) for (span, lab) in items if lab.endswith(str(b))]
        w = [span for (span, lab) in seq if lab.startswith("write")]
        r = [span for (span, lab) in seq if lab.startswith("reduce")]
        for k in range(len(r)):
            assert r[k][0] >= w[k][1]
            if k + 1 < len(w):
                assert w[k + 1][0] >= r[k][1]


def test_flush_without_submit_is_noop_and_single_buffer_serializes():
    p = Program(n_buffers=1)
    assert p.flush(1) == OK
    for _ in range(3):
        p.acquire(0, 1)
        p.write(1, 0)
        p.submit(0, [1])
    w = p.spans_of("write0")
    r = p.spans_of("reduce0")
    assert w[1][0] >= r[0][1] and w[2][0] >= r[1][1]


def check_reuse_ordered(p):
    """Every write of a buffer starts after that buffer's previous reduction
    ended, and every reduction starts after its bucket's write ended."""
    sp = p.replay()
    for b in (0, 1):
        w = [sp[(s, i)] for (lab, s, i) in p.work if lab == f"write{b}"]
        r = [sp[(s, i)] for (lab, s, i) in p.work if lab == f"reduce{b}"]
        for k in range(len(r)):
            assert r[k][0] >= w[k][1]
            if k + 1 < len(w):
                assert w[k + 1][0] >= r[k][1]


def test_waits_implied_by_a_flush_are_not_enqueued():
    # steps of five buckets over two buffers, each ended by a flush into the
    # producer stream: the first acquires of the next step are already ordered
    # after every reduction (the producer waited on the tail), so they enqueue
    # no wait; every other acquire still waits, and no write races a reduction
    p = Program()
    prod = 1
    per_step = []
    for step in range(3):
        before = len([w for w in p.waits if w[0] == prod])
        for i in range(5):
            b = i % 2
            assert p.acquire(b, prod) == OK
            p.write(prod, b)
            assert p.submit(b, [prod]) == OK
        assert p.flush(prod) == OK
        per_step.append(len([w for w in p.waits if w[0] == prod]) - before)
    check_reuse_ordered(p)
    # step 0: acquires of buckets 2, 3, 4 wait (buffers reused), plus the flush;
    # later steps: buckets 0 and 1 reuse buffers the flush already covered
    assert per_step == [4, 4, 4]
    first = Program()
    for i in range(5):
        first.acquire(i % 2, prod)
        first.write(prod, i % 2)
        first.submit(i % 2, [prod])
    first.flush(prod)
    n0 = len(first.waits)
    first.acquire(0, prod)
    first.acquire(1, prod)
    assert len(first.waits) == n0   # covered by the flush: nothing enqueued
    first.close()
    p.close()


def test_a_flush_into_another_stream_does_not_cover_the_producer():
    p = Program()
    for i in range(2):
        p.acquire(i, 1)
        p.write(1, i)
        p.submit(i, [1])
    p.flush(3)                      # the caller is stream 3, not the producer
    n = len(p.waits)
    p.acquire(0, 1)
    assert len(p.waits) == n + 1 and p.waits[-1][0] == 1
    p.write(1, 0)
    p.submit(0, [1])
    check_reuse_ordered(p)
    p.close()


def test_producer_on_the_reduction_stream_needs_no_events():
    # reductions on the caller's own stream: stream order covers every
    # dependency, so nothing is recorded and nothing waited on
    p = Program()
    for i in range(6):
        b = i % 2
        assert p.acquire(b, RED) == OK
        p.write(RED, b)
        assert p.submit(b, [RED]) == OK
    assert p.flush(RED) == OK
    assert p.waits == [] and p.records == []
    check_reuse_ordered(p)
    p.close()


def test_a_first_other_producer_waits_on_an_event_recorded_late():
    # steps on the reduction stream record no completion events; when another
    # stream then overwrites a buffer, the event is recorded at that point
    # (after every reduction so far) and the reuse stays ordered; from then on
    # completion events are recorded at submission again
    p = Program()
    for i in range(4):
        b = i % 2
        assert p.acquire(b, RED) == OK
        p.write(RED, b)
        assert p.submit(b, [RED]) == OK
    assert p.records == []
    for i in range(4):
        b = i % 2
        assert p.acquire(b, 1) == OK
        p.write(1, b)
        assert p.submit(b, [1]) == OK
    assert p.flush(1) == OK
    assert any(s == RED for (_, s) in p.records)
    check_reuse_ordered(p)
    p.close()
