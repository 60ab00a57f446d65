"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and rejects bad arguments before any HIP call (so these run on CPU).

Fake device addresses are plain integers; every call below either fails
validation or has no work, so nothing is ever launched.
"""
import ctypes
import os
import re

import pytest

import gradient_sync_zr_amd as zr
from conftest import ROOT

A = 0x7F0000000000  # a fake, 256-byte aligned device address


def declared_functions():
    text = open(os.path.join(ROOT, "include", "zr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_calls():
    names = declared_functions()
    for n in ("zr_flatten_bucket", "zr_reduce_scatter_avg", "zr_all_gather", "zr_allreduce",
              "zr_sched_create", "zr_sched_acquire", "zr_sched_submit_rs", "zr_sched_flush",
              "zr_sched_destroy", "zr_last_error", "zr_version", "zr_plan_buckets"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(zr.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(zr.EXPORTS)


def test_version():
    assert zr.zr_version() >= 100


def ranks(K, base=A, stride=1 << 30):
    return [base + r * stride for r in range(K)]


def rs(K=8, ins=None, in_dt=zr.ZR_BF16, N=1000, outs=None, out_dt=zr.ZR_FP32, shift=1, order=0):
    ins = ranks(K) if ins is None else ins
    outs = ranks(K, base=A + (1 << 40)) if outs is None else outs
    zr.zr_reduce_scatter_avg(ins, N, outs, chunk_shift=shift, average=True, order=order,
                             in_dtype=in_dt, out_dtype=out_dt, stream=0)


def expect(status, fn, *a, **kw):
    with pytest.raises(zr.ZrError) as e:
        fn(*a, **kw)
    assert e.value.status == status, str(e.value)
    assert zr.zr_last_error() != ""


@pytest.mark.parametrize("K", [0, -1, 65, 1000])
def test_rs_rejects_bad_k(K):
    lib = zr.lib()
    t = (ctypes.c_void_p * 64)(*ranks(64))
    st = lib.zr_reduce_scatter_avg(K, t, 0, 100, t, 1, 0, 1, 0, None)
    assert st == zr.ZR_ERR_INVALID


def test_rs_validation_errors():
    expect(zr.ZR_ERR_INVALID, rs, N=-1)
    expect(zr.ZR_ERR_UNSUPPORTED, rs, in_dt=2)
    expect(zr.ZR_ERR_UNSUPPORTED, rs, out_dt=7)
    expect(zr.ZR_ERR_INVALID, rs, shift=8)
    expect(zr.ZR_ERR_INVALID, rs, shift=-1)
    expect(zr.ZR_ERR_INVALID, rs, order=5)
    expect(zr.ZR_ERR_INVALID, rs, ins=[A] * 7 + [0])
    expect(zr.ZR_ERR_ALIGN, rs, ins=ranks(7) + [A + (7 << 30) + 1])       # odd bf16 address
    expect(zr.ZR_ERR_ALIGN, rs, in_dt=zr.ZR_FP32, ins=ranks(7) + [A + (7 << 30) + 2])
    expect(zr.ZR_ERR_ALIGN, rs, outs=ranks(7, base=A + (1 << 40)) + [A + (1 << 41) + 2])
    # two outputs overlapping: C = 125 fp32 = 500 bytes
    outs = ranks(8, base=A + (1 << 40), stride=256)
    expect(zr.ZR_ERR_ALIAS, rs, outs=outs)
    # an output inside an input
    expect(zr.ZR_ERR_ALIAS, rs, outs=[A + 64] + ranks(7, base=A + (1 << 40)))


def test_rs_rejects_unknown_flag_bits():
    lib = zr.lib()
    t = (ctypes.c_void_p * 8)(*ranks(8))
    o = (ctypes.c_void_p * 8)(*ranks(8, base=A + (1 << 40)))
    for flags in (4, 8, -1, 7):
        assert lib.zr_reduce_scatter_avg(8, t, 0, 100, o, 1, 1, flags, 0, None) == zr.ZR_ERR_INVALID
    for flags in (0, 1, 2, 3):   # valid flags, N = 0: no work, no HIP call
        assert lib.zr_reduce_scatter_avg(8, t, 0, 0, o, 1, 1, flags, 0, None) == zr.ZR_OK


def test_rs_duplicate_inputs_and_zero_n_are_accepted_without_work():
    rs(N=0)                                  # no work: OK before any HIP call
    rs(N=0, ins=[0] * 8, outs=[0] * 8)       # tables unused when N == 0


def test_allreduce_validation():
    lib = zr.lib()
    K = 4

    def call(ins, outs, dt=zr.ZR_BF16, N=64, fused=1, scratch=None, order=0):
        t_in = (ctypes.c_void_p * K)(*ins)
        t_out = (ctypes.c_void_p * K)(*outs)
        return lib.zr_allreduce(K, t_in, t_out, dt, N, 0, order, fused, scratch, None)

    ins = ranks(K)
    assert call(ins, ins, N=0) == zr.ZR_OK
    assert call(ins, ins, dt=3) == zr.ZR_ERR_UNSUPPORTED
    assert call(ins, ins, N=-5) == zr.ZR_ERR_INVALID
    assert call(ins, ins, order=9) == zr.ZR_ERR_INVALID
    # out[0] is in[1]: not the same rank -> alias
    assert call(ins, [ins[1], ins[0], ins[2], ins[3]]) == zr.ZR_ERR_ALIAS
    # out partly overlapping its own input
    assert call(ins, [ins[0] + 2] + ins[1:]) == zr.ZR_ERR_ALIAS
    # composed path needs scratch
    outs = ranks(K, base=A + (1 << 40))
    assert call(ins, outs, fused=0, scratch=None) == zr.ZR_ERR_INVALID
    assert call(ins, outs, fused=0, scratch=A + (1 << 41) + 1) == zr.ZR_ERR_ALIGN
    assert call(ins, outs, fused=0, scratch=ins[2]) == zr.ZR_ERR_ALIAS


def test_all_gather_validation():
    lib = zr.lib()
    K = 8

    def call(segs, shards=None, fulls=None, shift=0, dt=zr.ZR_BF16):
        s = (ctypes.c_void_p * K)(*(shards or ranks(K)))
        f = (ctypes.c_void_p * K)(*(fulls or ranks(K, base=A + (1 << 40))))
        arr = (zr.zr_seg * max(1, len(segs)))(*[zr.zr_seg(*x) for x in segs])
        return lib.zr_all_gather(K, s, f, dt, arr, len(segs), shift, None, 0, None)

    assert call([]) == zr.ZR_OK
    assert call([(0, 0, 0)]) == zr.ZR_OK
    assert call([(0, 0, 10)], shift=8) == zr.ZR_ERR_INVALID
    assert call([(0, 0, -1)]) == zr.ZR_ERR_INVALID
    assert call([(-1, 0, 10)]) == zr.ZR_ERR_INVALID
    assert call([(0, 0, 10)], dt=4) == zr.ZR_ERR_UNSUPPORTED
    assert call([(0, 0, 100), (50, 50, 100)]) == zr.ZR_ERR_ALIAS  # two segs write [50, 100)
    assert call([(0, 0, 10)], fulls=ranks(K, base=A + (1 << 40), stride=4)) == zr.ZR_ERR_ALIAS
    assert call([(0, 0, 10)], fulls=ranks(K)) == zr.ZR_ERR_ALIAS   # fulls == shards


def test_flatten_validation():
    lib = zr.lib()
    K, F = 2, 3

    def call(numels, padded, frags=None, buckets=None, dt=zr.ZR_BF16):
        fr = (ctypes.c_void_p * (K * F))(*(frags or ranks(K * F)))
        nm = (ctypes.c_int64 * F)(*numels)
        b = (ctypes.c_void_p * K)(*(buckets or ranks(K, base=A + (1 << 40))))
        return lib.zr_flatten_bucket(K, F, fr, nm, b, padded, dt, None, 0, None)

    assert call([0, 0, 0], 0) == zr.ZR_OK
    assert call([1, 2, 3], 5) == zr.ZR_ERR_INVALID          # padded < total
    assert call([1, -2, 3], 8) == zr.ZR_ERR_INVALID
    assert call([1, 2, 3], 8, dt=9) == zr.ZR_ERR_UNSUPPORTED
    assert call([1, 2, 3], 8, buckets=[A + (1 << 40), A + (1 << 40) + 4]) == zr.ZR_ERR_ALIAS
    frags = ranks(K * F)
    frags[4] = A + (1 << 40) + 2                               # fragment inside bucket 0
    assert call([1, 2, 3], 8, frags=frags) == zr.ZR_ERR_ALIAS
    frags = ranks(K * F)
    frags[1] = 0
    assert call([1, 2, 3], 8, frags=frags) == zr.ZR_ERR_INVALID


def test_overlap_checks_on_a_large_fragment_table():
    # 8 ranks x 500 fragments, laid end to end with every partition in a gap
    # between two fragments; the plan is validated and built on the host alone.
    # Partitions that touch their neighbours pass; one element of overlap with
    # any fragment, deep in the table or at either end, is an alias; an empty
    # fragment whose address lies inside a partition is ignored.
    lib = zr.lib()
    K, F = 8, 500
    numels = [2 * (1 + (p * 37) % 97) for p in range(F)]  # even: partitions stay 4-byte aligned
    N = -(-sum(numels) // K) * K + 16
    C = N // K
    addrs, cur = [], A
    outs = []
    for r in range(K):
        for p in range(F):
            addrs.append(cur)
            cur += numels[p] * 2             # bf16 fragments, back to back
            if p == 250:                     # a partition (fp32) in the middle of rank r's run
                outs.append(cur)
                cur += C * 4
    nm = (ctypes.c_int64 * F)(*numels)

    def plan(frags, o, numels_arr=nm):
        fr = (ctypes.c_void_p * (K * F))(*frags)
        ot = (ctypes.c_void_p * K)(*o)
        h = ctypes.c_void_p()
        st = lib.zr_rsf_plan_create(K, F, fr, numels_arr, N, 0, ot, 1, 1, 1, 0, None, 0, ctypes.byref(h))
        if st == zr.ZR_OK:
            assert lib.zr_rsf_plan_destroy(h) == zr.ZR_OK
        return st

    assert plan(addrs, outs) == zr.ZR_OK
    for r, delta in ((0, -4), (5, 4), (7, -4), (2, 4)):
        o = list(outs)
        o[r] = outs[r] + delta                # 4 bytes into fragment 250 or 251 of rank r
        assert plan(addrs, o) == zr.ZR_ERR_ALIAS, (r, delta)
    o = list(outs)
    o[3] = addrs[3 * F] - 4                   # over rank 2's last fragment and rank 3's first ones
    assert plan(addrs, o) == zr.ZR_ERR_ALIAS
    # an empty fragment whose address lies inside partition 2 is not a buffer
    nm0 = list(numels)
    nm0[499] = 0
    fr = list(addrs)
    fr[2 * F + 499] = outs[2] + 64
    assert plan(fr, outs, (ctypes.c_int64 * F)(*nm0)) == zr.ZR_OK


@pytest.mark.parametrize("entry", ["call", "plan"])
def test_reduce_scatter_frags_validation(entry):
    # the one-shot call and the plan share their validation; a valid plan is
    # built on the host alone, so it is created (and destroyed) here too
    lib = zr.lib()
    K, F = 2, 3

    def call(numels, N, frags=None, outs=None, flags=1, shift=1, order=0, in_dt=0, out_dt=1):
        fr = (ctypes.c_void_p * (K * F))(*(frags or ranks(K * F)))
        nm = (ctypes.c_int64 * F)(*numels)
        o = (ctypes.c_void_p * K)(*(outs or ranks(K, base=A + (1 << 40))))
        if entry == "call":
            return lib.zr_reduce_scatter_frags(K, F, fr, nm, N, in_dt, o, out_dt, shift, flags,
                                               order, None, 0, None)
        h = ctypes.c_void_p(1234)
        st = lib.zr_rsf_plan_create(K, F, fr, nm, N, in_dt, o, out_dt, shift, flags, order, None, 0,
                                    ctypes.byref(h))
        if st == zr.ZR_OK:
            if N == 0:
                assert lib.zr_rsf_plan_launch(h, None) == zr.ZR_OK  # launches nothing
            assert lib.zr_rsf_plan_destroy(h) == zr.ZR_OK
        else:
            assert not h.value  # nothing was handed out
        return st

    assert call([0, 0, 0], 0) == zr.ZR_OK
    if entry == "plan":
        for kw in ({}, dict(flags=3, order=2), dict(in_dt=1, out_dt=0, shift=0, order=1)):
            assert call([1, 2, 3], 8, **kw) == zr.ZR_OK
    assert call([1, 2, 3], 0) == zr.ZR_ERR_INVALID            # N < total
    assert call([1, 2, 3], 5) == zr.ZR_ERR_INVALID
    assert call([1, -2, 3], 8) == zr.ZR_ERR_INVALID
    assert call([1, 2, 3], 8, flags=4) == zr.ZR_ERR_INVALID
    assert call([1, 2, 3], 8, shift=2) == zr.ZR_ERR_INVALID
    assert call([1, 2, 3], 8, order=3) == zr.ZR_ERR_INVALID
    assert call([1, 2, 3], 8, in_dt=5) == zr.ZR_ERR_UNSUPPORTED
    frags = ranks(K * F)
    frags[2] = A + (1 << 40) + 8                              # fragment inside out[0]
    assert call([1, 2, 3], 8, frags=frags) == zr.ZR_ERR_ALIAS
    frags = ranks(K * F)
    frags[4] = 0
    assert call([1, 2, 3], 8, frags=frags) == zr.ZR_ERR_INVALID
    frags[4] = A + 1                                           # odd bf16 address
    assert call([1, 2, 3], 8, frags=frags) == zr.ZR_ERR_ALIGN
    assert call([1, 2, 3], 8, outs=[A + (1 << 40)] * 2) == zr.ZR_ERR_ALIAS


def greedy_reference(numels, cap):
    """The prefetch loop of the ZeRO-3 parameter coordinator as the page
    describes it (DeepSpeed ZeRO-3 源码解析, 2.1 step 3 and 2.2): keep taking
    the next parameter while the amount gathered so far is below the cap."""
    buckets, i = [], 0
    while i < len(numels):
        cur, total = [], 0
        while i < len(numels) and total < cap:
            cur.append(i)
            total += numels[i]
            i += 1
        buckets.append(cur)
    return buckets


@pytest.mark.parametrize("numels,cap", [
    ([5, 5, 5, 5], 10), ([100], 10), ([1, 100, 1], 10), ([], 3), ([0, 0, 4, 0], 4),
    ([3, 3, 3, 3, 3, 3, 3], 7), ([10, 1, 1, 10, 1], 10)])
def test_plan_buckets_matches_greedy_rule(numels, cap):
    got, nb = zr.zr_plan_buckets(numels, cap)
    ref = greedy_reference(numels, cap)
    assert nb == len(ref)
    for b, items in enumerate(ref):
        for i in items:
            assert got[i] == b


def test_plan_buckets_transformer_50mb():
    from synth import workloads as W
    ps = W.llama_like_params()
    cap = W.ZERO3["prefetch_bytes"] // W.ZERO3["elem_bytes"]
    got, nb = zr.zr_plan_buckets([p.numel for p in ps], cap)
    assert nb == 162
    assert nb == len(greedy_reference([p.numel for p in ps], cap))
    with pytest.raises(zr.ZrError):
        zr.zr_plan_buckets([1, 2], 0)
    with pytest.raises(zr.ZrError):
        zr.zr_plan_buckets([1, zr.ZR_MAX_ELEMS + 1], 10)


def test_header_constants_match_the_binding():
    text = open(os.path.join(ROOT, "include", "zr.h")).read()
    assert re.search(r"#define ZR_MAX_RANKS 64\b", text) and zr.ZR_MAX_RANKS == 64
    assert re.search(r"#define ZR_MAX_ELEMS \(1LL << 40\)", text) and zr.ZR_MAX_ELEMS == 1 << 40


def test_sizes_above_the_element_limit_are_rejected():
    # every size, offset and running total stays within ZR_MAX_ELEMS, so tile
    # numbers fit the kernels' 32 bits; rejected before any HIP call
    lib = zr.lib()
    big = zr.ZR_MAX_ELEMS
    K, F = 2, 3
    fr = (ctypes.c_void_p * (K * F))(*ranks(K * F))
    o = (ctypes.c_void_p * K)(*ranks(K, base=A + (1 << 41)))

    def flatten(numels, padded):
        nm = (ctypes.c_int64 * F)(*numels)
        return lib.zr_flatten_bucket(K, F, fr, nm, o, padded, zr.ZR_BF16, None, 0, None)

    def frags(numels, N):
        nm = (ctypes.c_int64 * F)(*numels)
        return lib.zr_reduce_scatter_frags(K, F, fr, nm, N, zr.ZR_BF16, o, zr.ZR_FP32, 1, 1, 0, None, 0,
                                           None)

    for fn in (flatten, frags):
        assert fn([1, big + 1, 3], big + 8) == zr.ZR_ERR_INVALID       # one fragment too large
        assert fn([big, 1, 0], big + 1) == zr.ZR_ERR_INVALID          # their total too large
        assert fn([1 << 62, 1 << 62, 1 << 62], 8) == zr.ZR_ERR_INVALID  # a total that would wrap
    assert flatten([1, 2, 3], big + 1) == zr.ZR_ERR_INVALID           # the padded bucket
    s = (ctypes.c_void_p * 8)(*ranks(8))
    f = (ctypes.c_void_p * 8)(*ranks(8, base=A + (1 << 41)))
    for seg in ((big + 1, 0, 10), (0, big + 1, 10), (0, 0, big + 1)):
        arr = (zr.zr_seg * 1)(zr.zr_seg(*seg))
        assert lib.zr_all_gather(8, s, f, zr.ZR_BF16, arr, 1, 0, None, 0, None) == zr.ZR_ERR_INVALID
    t = (ctypes.c_void_p * 8)(*ranks(8))
    assert lib.zr_reduce_scatter_avg(8, t, 0, big + 1, f, 1, 1, 1, 0, None) == zr.ZR_ERR_INVALID


def test_prefetch_config_validation():
    # every rejection happens before a HIP call, so it is visible without a GPU
    lib = zr.lib()
    K = 2
    numels = [100, 7]

    def create(**over):
        kw = dict(shard_offsets=[0, 50], shards=ranks(K), arenas=ranks(K, base=A + (1 << 40)),
                  arena_numel=1000, steps=[[0], [1]], bucket=10, max_live=100, reuse=0, ongoing=2,
                  shift=0, dtype=zr.ZR_BF16, K=K, numels=numels)
        kw.update(over)
        # stream handles are placeholders: a rejected config never reaches them
        c = zr._pf_config(kw["K"], kw["dtype"], kw["numels"], kw["steps"], kw["bucket"],
                          kw["max_live"], kw["arena_numel"], kw["ongoing"], kw["reuse"],
                          kw["shard_offsets"], kw["shards"], kw["arenas"], kw["shift"],
                          gather_stream=0, compute_stream=0)
        h = ctypes.c_void_p(77)
        st = lib.zr_pf_create(ctypes.byref(c), ctypes.byref(h))
        assert st == zr.ZR_OK or not h.value
        return st

    assert create(K=0) == zr.ZR_ERR_INVALID
    assert create(dtype=7) == zr.ZR_ERR_UNSUPPORTED
    assert create(numels=[100, 0]) == zr.ZR_ERR_INVALID
    assert create(arena_numel=0) == zr.ZR_ERR_INVALID
    assert create(shift=2) == zr.ZR_ERR_INVALID
    assert create(steps=[[0], [2]]) == zr.ZR_ERR_INVALID           # not a parameter id
    assert create(bucket=0) == zr.ZR_ERR_INVALID
    assert create(max_live=0) == zr.ZR_ERR_INVALID
    assert create(reuse=-1) == zr.ZR_ERR_INVALID
    assert create(ongoing=0) == zr.ZR_ERR_INVALID
    assert create(shard_offsets=[0, -1]) == zr.ZR_ERR_INVALID
    assert create(shards=[A, 0]) == zr.ZR_ERR_INVALID
    assert create(arenas=[A + (1 << 40) + 1, A + (1 << 41)]) == zr.ZR_ERR_ALIGN
    assert create(arenas=[A + (1 << 40)] * 2) == zr.ZR_ERR_ALIAS    # one arena for both ranks
    assert create(arenas=[A + 64, A + (1 << 41)]) == zr.ZR_ERR_ALIAS  # arena over rank 0's shards
    assert lib.zr_pf_create(None, ctypes.byref(ctypes.c_void_p())) == zr.ZR_ERR_INVALID
    assert lib.zr_pf_destroy(None) == zr.ZR_OK


def test_prefetch_plan_on_the_host():
    # zr_pf_plan needs no buffers: the same core run with gathers that finish
    # at once; a capacity that cannot hold a step is ZR_ERR_NOMEM
    numels = [40, 30, 20, 10]
    steps = [[0], [1, 2], [3], [2], [1], [0]]
    st = zr.zr_pf_plan(numels, steps, 30, 60, 1000, max_reuse_numel=25, iterations=2)
    assert st["live"] == 0 and st["peak_live"] <= 60 + 40 + 40
    assert st["immediate_gathers"] >= 2
    with pytest.raises(zr.ZrError) as e:
        zr.zr_pf_plan(numels, steps, 30, 60, 40, max_reuse_numel=0)  # step 1 needs 50
    assert e.value.status == zr.ZR_ERR_NOMEM


# ------------------------------------------------------------- workspaces
def test_workspace_bytes():
    # zero while a call's table fits one argument block: min(32, 256 / K)
    # fragments (and the all-gather's 32 segments); above that, room for the
    # largest of the three staged tables with n fragments (plus the padding
    # entry) and n + K (fragment, chunk) pieces, in whole 256-byte units
    f = zr.zr_workspace_bytes
    for K in (1, 2, 8, 16, 64):
        fit = min(32, 256 // K)
        assert f(K, 0) == 0 and f(K, fit) == 0
        b = f(K, fit + 1)
        assert b > 0 and b % 256 == 0
        n = 1000
        need_rsf = 8 * (n + K + 1) + ((12 * (n + K) + 7) // 8) * 8 + 16 * (n + 1) + 8 * K * (n + 1)
        need_flat = 8 * (n + 2) + 8 * (n + 1) + 16 * (n + 1) + 8 * K * (n + 1)
        need_ag = 8 * (n + 1) + 48 * n
        assert f(K, n) == -(-max(need_rsf, need_flat, need_ag) // 256) * 256
        assert f(K, n + 1) >= f(K, n)
    assert f(0, 100) == 0 and f(65, 100) == 0 and f(8, -1) == 0


def _frag_tables(K, F):
    fr = (ctypes.c_void_p * (K * F))(*[A + i * (1 << 24) for i in range(K * F)])
    nm = (ctypes.c_int64 * F)(*([1000] * F))
    o = (ctypes.c_void_p * K)(*ranks(K, base=A + (1 << 42), stride=1 << 24))
    return fr, nm, o


@pytest.mark.parametrize("entry", ["call", "plan", "flatten", "flatten_plan"])
def test_workspace_errors_come_before_any_work(entry):
    # a workspace too small for the staged table, misaligned, or overlapping
    # a buffer of the call is rejected on the host (no GPU here: a call that
    # got as far as staging would fail with ZR_ERR_HIP instead)
    lib = zr.lib()
    K, F = 64, 10
    fr, nm, o = _frag_tables(K, F)
    N = F * 1000 + 24
    ws_ok = A + (1 << 43)

    def call(ws, wsb):
        h = ctypes.c_void_p()
        if entry == "call":
            return lib.zr_reduce_scatter_frags(K, F, fr, nm, N, 0, o, 1, 1, 1, 0, ws, wsb, None)
        if entry == "plan":
            return lib.zr_rsf_plan_create(K, F, fr, nm, N, 0, o, 1, 1, 1, 0, ws, wsb, ctypes.byref(h))
        if entry == "flatten":
            return lib.zr_flatten_bucket(K, F, fr, nm, o, N, 0, ws, wsb, None)
        return lib.zr_flatten_plan_create(K, F, fr, nm, o, N, 0, ws, wsb, ctypes.byref(h))

    need = zr.zr_workspace_bytes(K, F)
    assert need > 0
    assert call(ws_ok, 64) == zr.ZR_ERR_WORKSPACE
    assert "workspace" in zr.zr_last_error()
    assert call(ws_ok + 4, need) == zr.ZR_ERR_ALIGN
    assert call(ws_ok, 0) == zr.ZR_ERR_WORKSPACE
    assert call(o[3], need) == zr.ZR_ERR_ALIAS          # the table would overwrite an output
    assert call(fr[5], need) == zr.ZR_ERR_ALIAS         # ... or a fragment


def test_all_gather_workspace_errors():
    lib = zr.lib()
    K, n = 8, 40
    s = (ctypes.c_void_p * K)(*ranks(K))
    f = (ctypes.c_void_p * K)(*ranks(K, base=A + (1 << 40)))
    segs = [(i * 100, i * 800, 800) for i in range(n)]
    arr = (zr.zr_seg * n)(*[zr.zr_seg(*x) for x in segs])
    ws = A + (1 << 43)
    assert lib.zr_all_gather(K, s, f, 0, arr, n, 0, ws, 64, None) == zr.ZR_ERR_WORKSPACE
    assert lib.zr_all_gather(K, s, f, 0, arr, n, 0, ws + 2, 1 << 20, None) == zr.ZR_ERR_ALIGN
    assert lib.zr_all_gather(K, s, f, 0, arr, n, 0, f[2], 1 << 20, None) == zr.ZR_ERR_ALIAS


@pytest.mark.parametrize("K,F", [(8, 32), (8, 33), (8, 64), (64, 4), (64, 5), (64, 300), (16, 100)])
def test_plans_without_workspace_count_their_launches(K, F):
    # without a workspace a plan takes min(32, 256 / K) fragments per launch
    # (the padding entry rides in a spare slot of the last one); plans are
    # built on the host, so the count is visible without a GPU
    fr, nm, o = _frag_tables(K, F)
    N = F * 1000 + K
    per = min(32, 256 // K)
    lib = zr.lib()
    for create, info, destroy, args in (
            (lib.zr_rsf_plan_create, lib.zr_rsf_plan_info, lib.zr_rsf_plan_destroy,
             (K, F, fr, nm, N, 0, o, 1, 1, 1, 0, None, 0)),
            (lib.zr_flatten_plan_create, lib.zr_flatten_plan_info, lib.zr_flatten_plan_destroy,
             (K, F, fr, nm, o, N, 0, None, 0))):
        h = ctypes.c_void_p()
        assert create(*args, ctypes.byref(h)) == zr.ZR_OK, zr.zr_last_error()
        n, b = ctypes.c_int(-1), ctypes.c_size_t(1)
        assert info(h, ctypes.byref(n), ctypes.byref(b)) == zr.ZR_OK
        assert n.value == -(-F // per) and b.value == 0
        assert destroy(h) == zr.ZR_OK


def test_rs_plan_validation_matches_the_call():
    # a plan is validated exactly as the one-shot call; N == 0 plans launch nothing
    lib = zr.lib()
    K = 8
    ins = (ctypes.c_void_p * K)(*ranks(K))
    outs = (ctypes.c_void_p * K)(*ranks(K, base=A + (1 << 40)))
    bad_outs = (ctypes.c_void_p * K)(*ranks(K, base=A + (1 << 40), stride=4))
    for N, o, shift, flags, want in ((1000, outs, 1, 1, zr.ZR_OK), (0, outs, 1, 1, zr.ZR_OK),
                                     (1000, bad_outs, 1, 1, zr.ZR_ERR_ALIAS), (1000, outs, 8, 1, zr.ZR_ERR_INVALID),
                                     (1000, outs, 1, 4, zr.ZR_ERR_INVALID), (-1, outs, 1, 1, zr.ZR_ERR_INVALID)):
        h = ctypes.c_void_p()
        st = lib.zr_rs_plan_create(K, ins, 0, N, o, 1, shift, flags, 0, ctypes.byref(h))
        assert st == want, (N, shift, flags, zr.zr_last_error())
        if st == zr.ZR_OK:
            if N == 0:
                assert lib.zr_rs_plan_launch(h, None) == zr.ZR_OK
            assert lib.zr_rs_plan_destroy(h) == zr.ZR_OK
        else:
            assert h.value is None


def _plan_in_child(env):
    # a reduce-scatter plan is built on the host (no GPU needed), which reads
    # the library's environment settings
    code = ("import ctypes, gradient_sync_zr_amd as zr\n"
            "lib = zr.lib(); K = 8; A = %d\n"
            "ins = (ctypes.c_void_p * K)(*[A + r * (1 << 30) for r in range(K)])\n"
            "outs = (ctypes.c_void_p * K)(*[A + (1 << 40) + r * (1 << 30) for r in range(K)])\n"
            "h = ctypes.c_void_p()\n"
            "assert lib.zr_rs_plan_create(K, ins, 0, 100000, outs, 1, 1, 1, 0, ctypes.byref(h)) == 0\n"
            "assert lib.zr_rs_plan_destroy(h) == 0\n" % A)
    import subprocess
    import sys
    return subprocess.run([sys.executable, "-c", code], env=dict(os.environ, **env), cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_force_path_setting_is_read_and_a_bad_value_reported():
    for value in ("element", "small", "large", "auto", ""):
        r = _plan_in_child({"ZR_FORCE_PATH": value, "ZR_DEBUG": "1"})
        assert r.returncode == 0, r.stderr
        assert "libzr:" not in r.stderr, (value, r.stderr)
    r = _plan_in_child({"ZR_FORCE_PATH": "vectorised"})
    assert r.returncode == 0, r.stderr
    assert "libzr: ZR_FORCE_PATH=vectorised is not one of element, small, large; ignored" in r.stderr
