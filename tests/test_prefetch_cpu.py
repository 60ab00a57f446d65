"""Prefetch coordinator logic on the CPU.

The coordinator core that libzr uses (prefetch_core.hpp) is compiled here
against a backend that only logs (tests/kit/pf_sim.cpp). A host program
walks a trace: fetch(t), the step's compute on the compute stream (reading
the arena ranges the coordinator reports), release(t). The log is replayed on
a discrete-event model of two streams, events and host time: a work item
starts when its stream reaches it and not before the host enqueued it, a
stream wait holds the stream until the captured record completes, and a host
sync moves the host clock to the synced record's completion. Event queries
are answered from the same replay at the current host time.

What is checked follows "DeepSpeed ZeRO-3 源码解析" 2.1, 2.2 and 2.4: the
three parts of a fetch, the prefetch cap min(max_live - live, bucket) with the
greedy rule, the limit of outstanding fetches, the conservative-release
window, and, from the streams' side, that no compute reads a parameter before
its gather ends and no gather overwrites arena memory a compute still reads.
"""
import ctypes
import os
import random

import numpy as np
import pytest

from conftest import ROOT

KIT = os.path.join(ROOT, "tests", "kit")
CREATE, DESTROY, RECORD, WAIT, SYNC, GATHER = 1, 2, 3, 4, 5, 6
OK, BAD_ARG, BAD_STATE, NO_MEMORY, BACKEND = range(5)
GS, CS = 1, 2  # gather and compute stream ids

QUERY = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_int)
_lib = None


def lib():
    global _lib
    if _lib is None:
        # PF_SIM_LIBRARY may name another build of the same simulator (the sanitizer
        # test runs this module against one)
        path = os.environ.get("PF_SIM_LIBRARY") or os.path.join(KIT, "libpf_sim.so")
        if not os.path.exists(path):
            import sys
            sys.path.insert(0, os.path.join(ROOT, "tests"))
            from kit import _build
            _build.build()
        L = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.pf_create.restype = vp
        L.pf_create.argtypes = [i32, vp, i32, vp, vp, vp, vp, QUERY, ctypes.POINTER(i32)]
        L.pf_fetch.argtypes = [vp, i32]
        L.pf_release.argtypes = [vp, i32]
        L.pf_offset.argtypes = [vp, i32]
        L.pf_offset.restype = i64
        L.pf_stats.argtypes = [vp, vp]
        L.pf_log_size.argtypes = [vp]
        L.pf_log_size.restype = i64
        L.pf_log.argtypes = [vp, vp]
        L.pf_destroy.argtypes = [vp]
        L.pf_shutdown.argtypes = [vp]
        _lib = L
    return _lib


class Run:
    """One coordinator, the host program driving it, and the replay."""

    def __init__(self, numels, steps, bucket, max_live, arena, max_reuse=0, max_ongoing=2,
                 align=1, g_per=1.0, c_per=2.0, serial=False, query="replay", fail_on_call=-1):
        self.numels = [int(n) for n in numels]
        self.steps = [list(s) for s in steps]
        self.max_live, self.max_ongoing, self.align = max_live, max_ongoing, align
        self.g_per, self.c_per = g_per, c_per
        self.gs, self.cs = (CS, CS) if serial else (GS, CS)
        self.query_mode = query
        off = np.cumsum([0] + [len(s) for s in self.steps]).astype(np.int32)
        flat = np.array([p for s in self.steps for p in s] or [0], dtype=np.int32)
        self._arrays = [np.array(self.numels, dtype=np.int64), off, flat,
                        np.array([bucket, max_live, max_reuse, arena, align], dtype=np.int64),
                        np.array([max_ongoing, self.gs, self.cs, fail_on_call], dtype=np.int32)]
        self._cb = QUERY(self._query)
        err = ctypes.c_int(-1)
        a = self._arrays
        self.h = lib().pf_create(len(self.numels), a[0].ctypes.data, len(self.steps), a[1].ctypes.data,
                                 a[2].ctypes.data, a[3].ctypes.data, a[4].ctypes.data, self._cb,
                                 ctypes.byref(err))
        self.init_err = err.value
        self.items = {GS: [], CS: []}   # (kind, payload, enqueue host time)
        self.host = 0.0
        self.version = {}
        self.seen = 0
        self.gathers = []    # dict(stream, idx, params=[(p, off)], host, step)
        self.computes = []   # dict(idx, step, reads=[(p, off, n)], host)
        self.live = {}       # param -> offset, after the last call
        self.fetch_step = None
        self.live_log = []   # (gather index, live before it)
        self.order = []      # ("g" | "c", index) in host order

    def close(self):
        lib().pf_destroy(self.h)

    # ---------------------------------------------------------- the log
    def _drain(self):
        n = lib().pf_log_size(self.h)
        if n == self.seen:
            return
        buf = np.zeros(n, dtype=np.int64)
        lib().pf_log(self.h, buf.ctypes.data)
        i = self.seen
        while i < n:
            op, a, b = (int(x) for x in buf[i:i + 3])
            i += 3
            if op == RECORD:
                v = self.version.get(a, 0) + 1
                self.version[a] = v
                self.items[b].append(("record", (a, v), self.host))
            elif op == WAIT:
                v = self.version.get(b, 0)
                if v:
                    self.items[a].append(("wait", (b, v), self.host))
            elif op == SYNC:
                v = self.version.get(a, 0)
                if v:
                    _, rec = self.replay()
                    self.host = max(self.host, rec[(a, v)])
            elif op == GATHER:
                pairs = [(int(buf[i + 2 * k]), int(buf[i + 2 * k + 1])) for k in range(b)]
                i += 2 * b
                dur = self.g_per * sum(self.numels[p] for p, _ in pairs)
                q = self.items[a]
                self.gathers.append(dict(stream=a, idx=len(q), params=pairs, host=self.host,
                                         step=self.fetch_step))
                self.order.append(("g", len(self.gathers) - 1))
                q.append(("work", ("gather", len(self.gathers) - 1), self.host, dur))
        self.seen = n

    def _query(self, ev):
        self._drain()
        v = self.version.get(ev, 0)
        if v == 0:
            return 1
        if self.query_mode == "never":
            return 0
        if self.query_mode == "always":
            return 1
        _, rec = self.replay()
        return 1 if rec[(ev, v)] <= self.host else 0

    def replay(self):
        """({(stream, idx): (start, end)} for work items, {record: time})."""
        pos = {s: 0 for s in self.items}
        t = {s: 0.0 for s in self.items}
        spans, rec = {}, {}
        progress = True
        while progress:
            progress = False
            for s, q in self.items.items():
                while pos[s] < len(q):
                    it = q[pos[s]]
                    kind, arg, enq = it[0], it[1], it[2]
                    if kind == "work":
                        start = max(t[s], enq)
                        spans[(s, pos[s])] = (start, start + it[3])
                        t[s] = start + it[3]
                    elif kind == "record":
                        rec[arg] = max(t[s], enq)
                    else:
                        if arg not in rec:
                            break
                        t[s] = max(t[s], rec[arg], enq)
                    pos[s] += 1
                    progress = True
        assert all(pos[s] == len(q) for s, q in self.items.items()), "streams deadlock"
        return spans, rec

    def _refresh_live(self):
        self.live = {}
        for p in range(len(self.numels)):
            o = lib().pf_offset(self.h, p)
            if o >= 0:
                self.live[p] = o

    # --------------------------------------------------- host program
    def fetch(self, t):
        self.fetch_step = t
        live0 = sum(self.numels[p] for p in self.live)
        g0 = len(self.gathers)
        st = lib().pf_fetch(self.h, t)
        self._drain()
        acc = live0
        for gi in range(g0, len(self.gathers)):
            self.live_log.append((gi, acc))
            acc += sum(self.numels[p] for p, _ in self.gathers[gi]["params"])
        self._refresh_live()
        return st

    def compute(self, t):
        reads = []
        for p in dict.fromkeys(self.steps[t]):
            assert p in self.live, f"step {t}: parameter {p} is not live at its compute"
            reads.append((p, self.live[p], self.numels[p]))
        q = self.items[self.cs]
        self.computes.append(dict(idx=len(q), step=t, reads=reads, host=self.host))
        self.order.append(("c", len(self.computes) - 1))
        q.append(("work", ("compute", t), self.host, self.c_per * sum(n for _, _, n in reads)))

    def release(self, t):
        st = lib().pf_release(self.h, t)
        self._drain()
        self._refresh_live()
        return st

    def walk(self, iterations=1):
        for _ in range(iterations):
            for t in range(len(self.steps)):
                assert self.fetch(t) == OK
                self.compute(t)
                assert self.release(t) == OK

    def stats(self):
        out = np.zeros(7, dtype=np.int64)
        lib().pf_stats(self.h, out.ctypes.data)
        keys = ("live", "peak_live", "gathers", "immediate_gathers", "host_syncs", "retained",
                "prefetch_trimmed")
        return dict(zip(keys, (int(x) for x in out)))

    # ------------------------------------------------------------ checks
    def rounded(self, n):
        return -(-n // self.align) * self.align

    def check(self):
        spans, _ = self.replay()
        gspan = [spans[(g["stream"], g["idx"])] for g in self.gathers]
        cspan = [spans[(self.cs, c["idx"])] for c in self.computes]
        last_writer = {}
        readers = []  # (compute index, arena range)
        for kind, i in self.order:
            if kind == "g":
                for p, off in self.gathers[i]["params"]:
                    lo, hi = off, off + self.rounded(self.numels[p])
                    # no compute still reading this memory when the gather writes it
                    for ci, (rlo, rhi) in readers:
                        if rlo < hi and lo < rhi:
                            assert cspan[ci][1] <= gspan[i][0] + 1e-9, \
                                f"gather {i} overwrites memory compute {ci} still reads"
                    last_writer[p] = i
            else:
                c = self.computes[i]
                for p, off, n in c["reads"]:
                    g = last_writer[p]
                    assert gspan[g][1] <= cspan[i][0] + 1e-9, \
                        f"compute of step {c['step']} starts before the gather of parameter {p}"
                    readers.append((i, (off, off + self.rounded(n))))
        # outstanding gathers when each is issued (the host's clock then);
        # meaningful when queries tell the truth ("always" claims every
        # gather finished, as the library's host plan does)
        if self.query_mode != "always":
            for i, g in enumerate(self.gathers):
                busy = sum(1 for k in range(i) if gspan[k][1] > g["host"] + 1e-9)
                assert busy <= self.max_ongoing - 1, f"gather {i}: {busy} gathers still outstanding"
        # live budget: a prefetch starts below max_live and overshoots by less than one parameter
        maxn = max(self.numels)
        for gi, live_before in self.live_log:
            g = self.gathers[gi]
            if set(p for p, _ in g["params"]) & set(self.steps[g["step"]]):
                continue  # part 1: what the step needs
            assert live_before < self.max_live
            after = live_before + sum(self.numels[p] for p, _ in g["params"])
            assert after < self.max_live + maxn
        return gspan, cspan


def batches(run):
    return [sorted(p for p, _ in g["params"]) for g in run.gathers]


def singletons(n):
    return [[p] for p in range(n)]


# ------------------------------------------------------------------ errors
def test_init_errors():
    good = dict(numels=[4, 4], steps=[[0], [1]], bucket=8, max_live=100, arena=64)
    r = Run(**good)
    assert r.init_err == OK
    r.close()
    for bad in (dict(numels=[4, 0]), dict(steps=[[0], [2]]), dict(bucket=0), dict(max_live=0),
                dict(max_reuse=-1), dict(max_ongoing=0)):
        r = Run(**{**good, **bad})
        assert r.init_err == BAD_ARG, bad
        r.close()
    r = Run(**{**good, "steps": [[0, 1]], "arena": 7})  # one step's parameters cannot fit
    assert r.init_err == NO_MEMORY
    r.close()
    r = Run(**good, fail_on_call=0)  # the first event creation fails
    assert r.init_err == BACKEND
    r.close()


def test_state_errors():
    r = Run([4, 4, 4], singletons(3), bucket=8, max_live=100, arena=64)
    assert r.fetch(1) == BAD_STATE       # out of trace order
    assert r.release(0) == BAD_STATE     # not fetched
    assert r.fetch(3) == BAD_ARG and r.fetch(-1) == BAD_ARG
    assert r.fetch(0) == OK
    assert r.fetch(0) == BAD_STATE       # fetched twice
    r.compute(0)
    assert r.release(0) == OK
    assert r.release(0) == BAD_STATE     # released twice
    r.close()


# ------------------------------------------------------- the caps (2.1, 2.2)
def test_prefetch_takes_the_next_parameters_up_to_the_bucket():
    # bucket 8: after step 0 the prefetch takes p1 (4) and p2 (4, reaching 8);
    # after step 1 it takes p3 (4) and p4 (7, crossing 8); then p5
    r = Run([10, 4, 4, 4, 7, 3], singletons(6), bucket=8, max_live=100, arena=1000)
    r.walk()
    assert batches(r) == [[0], [1, 2], [3, 4], [5]]
    assert r.stats()["immediate_gathers"] == 1
    r.walk()  # the next pass: step 0 again at once, the same prefetches
    assert batches(r)[4:] == [[0], [1, 2], [3, 4], [5]]
    r.check()
    r.close()


@pytest.mark.parametrize("max_live,want", [
    (12, [[0], [1, 2], [3], [4], [5], [6], [7], [8], [9]]),   # cap 7 then 2: one crossing param
    (10, [[0], [1], [2], [3], [4], [5], [6], [7], [8], [9]]),  # cap 5: exactly one param
    (5, [[0], [1], [2], [3], [4], [5], [6], [7], [8], [9]]),   # cap 0: nothing prefetched
])
def test_live_budget_bounds_the_prefetch(max_live, want):
    r = Run([5] * 10, singletons(10), bucket=100, max_live=max_live, arena=1000)
    r.walk()
    assert batches(r) == want
    st = r.stats()
    assert st["immediate_gathers"] == (10 if max_live == 5 else 1)
    assert st["peak_live"] == {12: 15, 10: 10, 5: 5}[max_live]
    r.check()
    r.close()


def test_outstanding_gathers_are_capped_and_the_host_blocks():
    # gathers that never report finished: the host syncs on the oldest
    for cap in (1, 2, 3):
        r = Run([3] * 12, singletons(12), bucket=3, max_live=1000, arena=1000, max_ongoing=cap,
                query="never", g_per=5.0, c_per=1.0)
        r.walk()
        st = r.stats()
        assert st["host_syncs"] > 0
        r.check()
        r.close()


# ------------------------------------------------------ conservative release
def expected_release(steps, numels, max_reuse):
    """The release sets written out from the page's rule (2.4)."""
    out = []
    for s, ps in enumerate(steps):
        rel = set(ps)
        seen = 0
        for t in range(s + 1, len(steps)):
            if seen >= max_reuse:
                break
            for q in steps[t]:
                rel.discard(q)
                seen += numels[q]
        out.append(rel)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_release_keeps_what_is_reused_within_the_window(seed):
    rng = random.Random(seed)
    n = rng.randint(2, 12)
    numels = [rng.randint(1, 50) for _ in range(n)]
    steps = [rng.sample(range(n), rng.randint(1, min(3, n))) for _ in range(rng.randint(3, 25))]
    reuse = rng.choice([0, 1, 30, 100, 10 ** 6])
    r = Run(numels, steps, bucket=rng.randint(1, 80), max_live=rng.randint(1, 200),
            arena=4 * sum(numels), max_reuse=reuse)
    want = expected_release(steps, numels, reuse)
    retained = 0
    for t in range(len(steps)):
        assert r.fetch(t) == OK
        r.compute(t)
        assert r.release(t) == OK
        for p in set(steps[t]):
            assert (p not in r.live) == (p in want[t]), (t, p)
        retained += len(set(steps[t]) - want[t])
    assert r.stats()["retained"] == retained
    assert not r.live  # nothing survives the end of the pass
    r.check()
    r.close()


# -------------------------------------------------------------- no races
@pytest.mark.parametrize("seed", range(40))
def test_random_traces_have_no_stream_races(seed):
    rng = random.Random(1000 + seed)
    n = rng.randint(3, 30)
    numels = [rng.randint(1, 1000) for _ in range(n)]
    steps = [rng.sample(range(n), rng.randint(1, min(3, n))) for _ in range(rng.randint(5, 60))]
    r = Run(numels, steps, bucket=rng.randint(1, 3000), max_live=rng.randint(1, 5000),
            arena=2 * sum(numels) + 1000, max_reuse=rng.choice([0, 500, 3000]),
            max_ongoing=rng.choice([1, 2, 2, 3]), align=rng.choice([1, 8]),
            g_per=1.0, c_per=rng.choice([0.3, 1.0, 3.0]), serial=rng.random() < 0.2,
            query=rng.choice(["replay", "never"]))
    r.walk(iterations=rng.randint(1, 3))
    r.check()
    assert r.stats()["live"] == 0
    r.close()


def test_destroy_waits_for_the_outstanding_gathers():
    # the host never sees a gather finish, so the last ones are still writing
    # the arena when the coordinator goes away: destroy blocks on each first
    r = Run([100] * 8, [[p] for p in range(8)], bucket=200, max_live=10_000, arena=10_000,
            query="never", g_per=10.0)
    for t in range(3):
        assert r.fetch(t) == OK
        r.compute(t)
        assert r.release(t) == OK
    spans, _ = r.replay()
    gather_end = max(spans[(g["stream"], g["idx"])][1] for g in r.gathers)
    assert r.host < gather_end
    lib().pf_shutdown(r.h)
    r._drain()
    assert r.host >= gather_end
    r.close()


def test_the_replay_catches_a_race():
    # if queries claimed unfinished gathers done, the coordinator would skip
    # the compute stream's waits: the checks must see that as a race. Each
    # prefetch takes two steps ahead, so the gather of [3, 4] is retired (by
    # the false answer) before step 3 would wait on it
    r = Run([50] * 8, singletons(8), bucket=100, max_live=1000, arena=1000, query="always",
            g_per=10.0, c_per=1.0)
    r.walk()
    with pytest.raises(AssertionError, match="starts before the gather"):
        r.check()
    r.close()


def test_arena_too_small_for_the_whole_prefetch_trims_it():
    # room for three parameters: prefetches are cut to what fits and resume later
    r = Run([4] * 8, singletons(8), bucket=100, max_live=100, arena=12)
    r.walk(iterations=2)
    st = r.stats()
    assert st["prefetch_trimmed"] > 0
    assert st["immediate_gathers"] == 2  # step 0 of each pass only
    r.check()
    r.close()


# --------------------------------------------------------------- overlap
def transformer_trace(layers=4, scale=10_000):
    from synth import workloads as W
    ps = W.llama_like_params(layers=layers)
    numels = [max(1, p.numel // scale) for p in ps]
    fwd = singletons(len(ps))
    return numels, fwd + fwd[::-1]


def compute_idle(r, cspan):
    idle = 0.0
    for a, b in zip(cspan, cspan[1:]):
        idle += max(0.0, b[0] - a[1])
    return idle


def test_gathers_hide_behind_longer_compute():
    numels, steps = transformer_trace()
    kw = dict(bucket=2500, max_live=100_000, arena=400_000, max_reuse=100_000, g_per=1.0, c_per=2.0)
    r = Run(numels, steps, **kw)
    r.walk()
    gspan, cspan = r.check()
    # after the first step's gather the compute stream never waits
    assert compute_idle(r, cspan) == 0.0
    total = cspan[-1][1]
    assert total == pytest.approx(gspan[0][1] + sum(b - a for a, b in cspan))
    r.close()
    s = Run(numels, steps, serial=True, **kw)  # one stream: nothing overlaps
    s.walk()
    gs, cs = s.check()
    gather_time = sum(b - a for a, b in gs)
    assert cs[-1][1] == pytest.approx(gather_time + sum(b - a for a, b in cs))
    # overlap saves every gather but the first
    assert cs[-1][1] - total == pytest.approx(gather_time - (gspan[0][1] - gspan[0][0]))
    s.close()


# ------------------------------------------------- the library's host plan
def test_library_plan_matches_the_core_here():
    import gradient_sync_zr_amd as zr
    numels, steps = transformer_trace(layers=8, scale=1000)
    kw = dict(bucket=25_000, max_live=1_000_000, arena=1_500_000, max_reuse=1_000_000)
    r = Run(numels, steps, align=128, query="always", **kw)
    r.walk(iterations=2)
    mine = r.stats()
    r.close()
    got = zr.zr_pf_plan(numels, steps, kw["bucket"], kw["max_live"], kw["arena"],
                        max_reuse_numel=kw["max_reuse"], iterations=2)
    for k in ("peak_live", "gathers", "immediate_gathers", "retained", "prefetch_trimmed"):
        assert got[k] == mine[k], k
    assert got["live"] == 0
