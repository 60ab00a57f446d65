"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test ties one part of the oracle to the pages' worked examples, to a
closed form, to brute force, or to an independent library routine, so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.

Sources are cited by page title and section:
  "图解 Ring All-Reduce" (the 4-GPU walkthrough): Phase 1 / Phase 2 tables.
  CMU 11-868 lecture 14 notes: section 2.2 (identities), 3.2 (ring rounds,
  placement, send volume), 3.3 (ring order vs a plain sum), 4.1 (average),
  exercise 3 / 4 answers.
  "DeepSpeed ZeRO-3 源码解析": section 5.1 (flat bucket offsets).
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import GOLDEN


# ------------------------------------------------------------------ helpers
def parse_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, *cells = [c.strip() for c in line.split("|")]
            phase, rnd, dev = head.split()
            rows.append((phase, int(rnd), int(dev), cells))
    return rows


def symbolic_inputs(K):
    """x_r[c] = 2^(K*r + c): every partial sum's bits name its addend set."""
    x = np.zeros((K, K), dtype=np.float32)
    for r in range(K):
        for c in range(K):
            x[r, c] = np.float32(2.0 ** (K * r + c))
    return x


def decode(value, K):
    v = int(value)
    assert v == value
    names = set()
    for r in range(K):
        for c in range(K):
            if v >> (K * r + c) & 1:
                names.add(f"{'abcd'[r]}{c}")
    return names


def check_golden(name, K):
    rows = parse_golden(name)
    checked = 0
    for phase, rnd, dev, cells in rows:
        n_rs = rnd if phase == "RS" else K - 1
        n_ag = rnd if phase == "AG" else 0
        state, _ = oracle.ring_run(symbolic_inputs(K), n_rs, n_ag)
        assert len(cells) == K
        for c, cell in enumerate(cells):
            if cell == ".":
                continue
            want = set(cell.split("+"))
            got = decode(state[dev, c, 0], K)
            assert got == want, f"{name}: {phase} round {rnd} device {dev} chunk {c}"
            checked += 1
    return checked


# ------------------------------------------------------- ring round tables
def test_ring_sim_matches_4gpu_walkthrough():
    # every written cell of the six tables of the 4-GPU walkthrough
    assert check_golden("ring4_walkthrough.txt", 4) == 48 + 36


def test_ring_sim_matches_3device_exercise():
    assert check_golden("ring3_exercise.txt", 3) > 15


@pytest.mark.parametrize("K", list(range(1, 24)))
def test_ring_placement_rank_holds_next_chunk(K):
    # lecture 14, 3.2: after K-1 scatter-reduce rounds rank r holds the full
    # sum of chunk (r+1) mod K, and no other cell is complete.
    x = np.zeros((K, K), dtype=np.float32)
    for r in range(K):
        x[r, :] = np.float32(2.0 ** r)
    state, _ = oracle.ring_run(x, K - 1, 0)
    full = np.float32(2.0 ** K - 1)
    for r in range(K):
        for c in range(K):
            is_full = state[r, c, 0] == full
            assert is_full == (c == (r + 1) % K) or K == 1


@pytest.mark.parametrize("K", list(range(1, 17)))
@pytest.mark.parametrize("C", [1, 3])
def test_send_volume_closed_form(K, C):
    # lecture 14, 3.2 and exercise 4: every device sends 2(K-1) chunks,
    # i.e. 2(K-1)/K * N elements with N = K*C.
    x = np.ones((K, K * C), dtype=np.float32)
    _, sent = oracle.ring_run(x, K - 1, K - 1)
    N = K * C
    assert all(int(s) == 2 * (K - 1) * N // K for s in sent)
    _, sent_rs = oracle.ring_run(x, K - 1, 0)
    assert all(int(s) == (K - 1) * C for s in sent_rs)


@pytest.mark.parametrize("K", [1, 2, 3, 4, 7, 8, 13, 16])
def test_allreduce_all_ranks_identical_and_exact(K):
    # 4-GPU walkthrough round 2.3: every GPU ends with the same sums.
    # Integer inputs keep every partial sum exact, so int64 brute force decides.
    rng = np.random.default_rng(K)
    C = 5
    xi = rng.integers(-8, 9, size=(K, K * C))
    state, _ = oracle.ring_run(xi.astype(np.float32), K - 1, K - 1)
    want = xi.sum(axis=0).reshape(K, C)
    for r in range(K):
        assert np.array_equal(state[r], want.astype(np.float32))


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 7, 8, 16])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_allreduce_average_is_the_exact_sum_over_k(K, dt):
    # SUM then divide by the world size (lecture 14, 4.1). Integer inputs make
    # the sum exact; for power-of-two K the quotient is exact as well, and for
    # other K the correctly rounded fp32 quotient equals rounding the fp64
    # quotient (s/K has a periodic binary expansion, never within fp64
    # precision of an fp32 midpoint). A bf16 output is one rounding of it.
    rng = np.random.default_rng(100 + K)
    C = 7
    N = K * C - (1 if K > 1 else 0)
    xi = rng.integers(-8, 9, size=(K, K * C))
    xi[:, N:] = 0
    want32 = (xi.sum(axis=0).astype(np.float64) / K).astype(np.float32)[:N]
    if dt == "f32":
        ins = [xi[r].astype(np.float32) for r in range(K)]
        want = want32
    else:
        ins = [oracle.f32_to_bf16(xi[r].astype(np.float32)) for r in range(K)]
        want = oracle.f32_to_bf16(want32)
    out = oracle.allreduce(ins, N, average=True)
    for r in range(K):
        assert np.array_equal(out[r][:N].view(want.dtype), want), (K, dt, r)


# ------------------------------------------------------------ direct fold
def wide_random(shape, rng):
    """fp32 values spread over many binades with both signs, so that the
    order of fp32 additions changes the rounded result."""
    mant = rng.integers(1 << 23, 1 << 24, size=shape).astype(np.float64)
    exp = rng.integers(-30, 8, size=shape)
    sign = rng.choice([-1.0, 1.0], size=shape)
    return (sign * mant * np.exp2(exp - 23)).astype(np.float32)


@pytest.mark.parametrize("K", list(range(1, 17)))
def test_fold_equals_ring_sim_bit_exact(K):
    rng = np.random.default_rng(100 + K)
    C = 37
    x = wide_random((K, K * C), rng)
    state, _ = oracle.ring_run(x, K - 1, 0)
    for j in range(K):
        xs = x[:, j * C:(j + 1) * C]
        got = oracle.fold_points(xs, np.full(C, j))
        holder = (j - 1) % K
        assert np.array_equal(got.view(np.uint32), state[holder, j].view(np.uint32))


@pytest.mark.parametrize("K", [3, 4, 8])
def test_reduce_scatter_equals_ring_sim(K):
    rng = np.random.default_rng(7 * K)
    C = 11
    x = wide_random((K, K * C), rng)
    state, _ = oracle.ring_run(x, K - 1, 0)
    out = oracle.reduce_scatter([x[r] for r in range(K)], K * C, np.float32, shift=1,
                                average=False)
    for r in range(K):
        assert np.array_equal(out[r].view(np.uint32),
                              state[r, (r + 1) % K].view(np.uint32))
    out0 = oracle.reduce_scatter([x[r] for r in range(K)], K * C, np.float32, shift=0,
                                 average=False)
    for r in range(K):
        assert np.array_equal(out0[r].view(np.uint32), out[(r - 1) % K].view(np.uint32))


def test_fold_order_handworked():
    """Two hand-derived cases (fp32 round-to-nearest-even) where only the ring
    order starting at the chunk's own rank gives the listed result.

    Case A, ranks 0..3 hold (1, e, e, -1) with e = 2^-24 at every index:
      start 0: 1+e ties to 1, again 1, then 1-1 -> 0
      start 1: e+e = 2e, 2e-1 exact, +1 -> 2e
      start 2: e-1 exact, +1 -> e, +e -> 2e
      start 3: -1+1 = 0, +e, +e -> 2e
    Case B, ranks 0..3 hold (1, e, -1, e):
      start 0: 1+e ties to 1, -1 -> 0, +e -> e
      start 1: e-1 exact, +e -> 2e-1 exact, +1 -> 2e
      start 2: -1+e exact, +1 -> e, +e -> 2e
      start 3: e+1 ties to 1, +e -> 1, -1 -> 0
    A plain rank-order sum gives 0 in case A for every chunk.
    """
    e = 2.0 ** -24
    K = 4
    for vals, want in (((1.0, e, e, -1.0), (0.0, 2 * e, 2 * e, 2 * e)),
                       ((1.0, e, -1.0, e), (e, 2 * e, 2 * e, 0.0))):
        N = 4 * 3
        ins = [np.full(N, v, dtype=np.float32) for v in vals]
        out = oracle.reduce_scatter(ins, N, np.float32, shift=1, average=False)
        for j in range(K):
            holder = (j - 1) % K
            assert np.all(out[holder] == np.float32(want[j])), (vals, j)
        avg = oracle.reduce_scatter(ins, N, np.float32, shift=1, average=True)
        for j in range(K):
            assert np.all(avg[(j - 1) % K] == np.float32(want[j] / 4))
    plain = np.float32(1.0) + np.float32(e) + np.float32(e) + np.float32(-1.0)
    assert plain == 0.0


def test_fold_equals_exact_sum_when_exact():
    # small integers in bf16: every partial sum is exact in fp32, so the fold
    # must equal the mathematical sum (fsum) whatever the order
    rng = np.random.default_rng(5)
    K, n = 64, 1000
    xi = rng.integers(-128, 129, size=(K, n))
    xs = xi.astype(np.float32)
    got = oracle.fold_points(xs, rng.integers(0, K, size=n))
    assert np.array_equal(got, xi.sum(axis=0).astype(np.float32))
    ex, ab = oracle.exact_sum_points(xs)
    assert np.array_equal(ex, xi.sum(axis=0).astype(np.float64))
    assert np.array_equal(ab, np.abs(xi).sum(axis=0).astype(np.float64))


def test_exact_sum_close_to_fsum():
    rng = np.random.default_rng(6)
    K, n = 64, 200
    xs = wide_random((K, n), rng)
    ex, ab = oracle.exact_sum_points(xs)
    for p in range(n):
        f = math.fsum(float(v) for v in xs[:, p])
        assert abs(ex[p] - f) <= K * 2.0 ** -52 * ab[p]


def test_ring_order_differs_from_plain_sum_but_within_tolerance():
    # lecture 14, 3.3: the ring's summation order differs from a plain sum in
    # the last bits (about 1e-5 relative at K = 64 in fp32).
    rng = np.random.default_rng(64)
    K, n = 64, 4096
    xs = rng.standard_normal((K, n)).astype(np.float32)
    ring = oracle.fold_points(xs, np.full(n, 5))
    plain = np.zeros(n, dtype=np.float32)
    for r in range(K):
        plain = plain + xs[r]
    assert np.any(ring != plain)
    ex, ab = oracle.exact_sum_points(xs)
    assert np.all(np.abs(ring.astype(np.float64) - ex) <= 1e-5 * ab)


# -------------------------------------------------------- reduce-scatter
@pytest.mark.parametrize("N,K", [(10, 4), (1, 8), (7, 8), (0, 3), (17, 16), (65, 64)])
def test_rs_ragged_tail_zero_padding(N, K):
    rng = np.random.default_rng(N * 131 + K)
    xi = rng.integers(-8, 9, size=(K, max(N, 1)))
    ins = [xi[r].astype(np.float32) for r in range(K)]
    out = oracle.reduce_scatter(ins, N, np.float32, shift=1, average=False)
    C = -(-N // K)
    total = xi.sum(axis=0)
    for q in range(K):
        j = (q + 1) % K
        for o in range(C):
            g = j * C + o
            if g < N:
                assert out[q][o] == total[g]
            else:
                assert out[q][o].view(np.uint32) == 0  # +0.0, sign bit clear


@pytest.mark.parametrize("K", [2, 3, 4, 5, 8, 64])
def test_average_is_sum_over_k(K):
    # lecture 14, 4.1: SUM then divide by the world size (one IEEE divide in
    # fp32, as numpy performs it); for power-of-two K it equals x(1/K).
    rng = np.random.default_rng(K)
    N = K * 9 + 3
    ins = [wide_random(N, rng) for _ in range(K)]
    s = oracle.reduce_scatter(ins, N, np.float32, shift=0, average=False)
    a = oracle.reduce_scatter(ins, N, np.float32, shift=0, average=True)
    for q in range(K):
        assert np.array_equal(a[q], s[q] / np.float32(K))
        if K & (K - 1) == 0:
            assert np.array_equal(a[q], s[q] * np.float32(1.0 / K))


def test_bf16_out_rounds_once():
    rng = np.random.default_rng(9)
    K, N = 8, 8 * 50
    ins = [oracle.f32_to_bf16(wide_random(N, rng)) for _ in range(K)]
    f = oracle.reduce_scatter(ins, N, np.float32, shift=1, average=True)
    b = oracle.reduce_scatter(ins, N, np.uint16, shift=1, average=True)
    for q in range(K):
        assert np.array_equal(b[q], torch_bf16_round(f[q]))


# ------------------------------------------------------------- all-gather
@pytest.mark.parametrize("K,shift", [(1, 0), (4, 0), (4, 1), (8, 0), (8, 3), (5, 2)])
def test_all_gather_rebuilds_original(K, shift):
    # ZeRO-3 parameter lifecycle: shards of 1/K are gathered back into the full
    # tensor; chunk j of the full tensor is the shard of rank (j - shift) mod K.
    rng = np.random.default_rng(K * 10 + shift)
    sizes = [1, 7, K * 3, 50, 2 * K + 1]
    Ws = [rng.integers(0, 65535, size=n).astype(np.uint16) for n in sizes]
    shard_len = sum(-(-n // K) for n in sizes)
    shards = [np.zeros(shard_len, dtype=np.uint16) for _ in range(K)]
    segs, soff, foff = [], 0, 0
    for W in Ws:
        n = W.size
        C = -(-n // K)
        padded = np.zeros(K * C, dtype=np.uint16)
        padded[:n] = W
        for j in range(K):
            shards[(j - shift) % K][soff:soff + C] = padded[j * C:(j + 1) * C]
        segs.append((soff, foff, n))
        soff += C
        foff += n
    fulls = [np.full(foff, 0xDEAD, dtype=np.uint16) for _ in range(K)]
    oracle.all_gather(shards, fulls, segs, shift)
    want = np.concatenate(Ws)
    for r in range(K):
        assert np.array_equal(fulls[r], want)


@pytest.mark.parametrize("K,N,dt", [(4, 16, np.float32), (8, 100, np.uint16),
                                    (3, 10, np.float32), (16, 33, np.uint16),
                                    (1, 7, np.uint16), (2, 1, np.float32)])
def test_allreduce_equals_ring_sim_and_rs_then_ag(K, N, dt):
    # lecture 14, 2.2: all-reduce = reduce-scatter then all-gather; the literal
    # ring (both phases) must give the same numbers on every rank.
    rng = np.random.default_rng(K + N)
    x = wide_random((K, N), rng)
    if dt == np.uint16:
        x = oracle.bf16_to_f32(oracle.f32_to_bf16(x))
    ins = [x[r].astype(np.float32) if dt == np.float32 else oracle.f32_to_bf16(x[r])
           for r in range(K)]
    out = oracle.allreduce(ins, N, average=False)
    C = -(-N // K)
    xp = np.zeros((K, K * C), dtype=np.float32)
    xp[:, :N] = x
    state, _ = oracle.ring_run(xp, K - 1, K - 1)
    ring = state[0].reshape(-1)[:N]
    want = ring if dt == np.float32 else torch_bf16_round(ring)
    for r in range(K):
        assert np.array_equal(out[r].view(np.uint8), np.asarray(want).view(np.uint8))
    # composition through the public RS and AG of the oracle
    sh = oracle.reduce_scatter(ins, N, dt, shift=1 % K, average=False)
    fulls = [np.zeros(N, dtype=dt) for _ in range(K)]
    oracle.all_gather(sh, fulls, [(0, 0, N)], shift=1 % K)
    for r in range(K):
        assert np.array_equal(fulls[r].view(np.uint8), out[r].view(np.uint8))


# ---------------------------------------------------------------- flatten
def test_flatten_is_concatenation_plus_zero_pad():
    # ZeRO-3 5.1: each grad lands at the running offset of the flat buffer.
    rng = np.random.default_rng(3)
    K, sizes = 3, [5, 1, 0, 17, 64]
    frags = [[rng.integers(1, 65535, size=n).astype(np.uint16) for n in sizes]
             for _ in range(K)]
    total = sum(sizes)
    padded = total + 6
    b = oracle.flatten(frags, sizes, padded)
    for r in range(K):
        want = np.concatenate(frags[r] + [np.zeros(6, dtype=np.uint16)])
        assert np.array_equal(b[r], want)


# ------------------------------------------------------------ bf16 codec
def torch_bf16_round(f32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def exact_bf16_round(x: float) -> int:
    """Round a finite float to bf16 by exact rational arithmetic: the textbook
    definition (nearest representable, ties to even significand)."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    v = Fraction(abs(x))
    e = math.frexp(abs(x))[1]  # abs(x) = m * 2^e with m in [0.5, 1)
    # direct construction: quantum at this binade
    E = max(e - 1, -126)          # unbiased exponent of the leading bit
    quantum = Fraction(2) ** (E - 7)
    k = v / quantum
    lo = math.floor(k)
    rem = k - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    mag = lo * quantum
    # encode magnitude
    if mag >= Fraction(2) ** 128:
        return sign | 0x7F80
    if mag < Fraction(2) ** -126:
        frac = int(mag / Fraction(2) ** -133)
        return sign | frac
    ex = math.floor(math.log2(mag))
    while Fraction(2) ** ex > mag:
        ex -= 1
    while Fraction(2) ** (ex + 1) <= mag:
        ex += 1
    frac = int((mag / Fraction(2) ** ex - 1) * 128)
    return sign | ((ex + 127) << 7) | frac


def test_bf16_widen_matches_torch_exhaustive():
    import torch
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_round_trip_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(h)
    back = oracle.f32_to_bf16(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], h[~nan])
    assert np.all(np.isnan(oracle.bf16_to_f32(back[nan])))


def test_bf16_round_matches_exact_rational_and_torch():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    # force ties and near-ties on both parities
    ties = (rng.integers(0, 2 ** 16, size=4000, dtype=np.uint64).astype(np.uint32) << 16) \
        | np.uint32(0x8000)
    near = ties + np.uint32(1)
    below = ties - np.uint32(1)
    special = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001, 0x00008000,
                        0x00018000, 0x80008000, 0x7F800000, 0xFF800000, 0x00000000,
                        0x80000000], dtype=np.uint32)
    allbits = np.concatenate([bits, ties, near, below, special])
    f = allbits.view(np.float32)
    finite = np.isfinite(f)
    ours = oracle.f32_to_bf16(f)
    tref = torch_bf16_round(f)
    assert np.array_equal(ours[finite], tref[finite])
    for v, o in zip(f[finite][:6000].tolist(), ours[finite][:6000].tolist()):
        assert exact_bf16_round(v) == o, hex(struct.unpack("<I", struct.pack("<f", v))[0])
    nanbits = np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7FBFFFFF], dtype=np.uint32)
    nb = oracle.f32_to_bf16(nanbits.view(np.float32))
    assert np.all(np.isnan(oracle.bf16_to_f32(nb)))
    inf = oracle.f32_to_bf16(np.array([np.inf, -np.inf], dtype=np.float32))
    assert inf.tolist() == [0x7F80, 0xFF80]


# ----------------------------------------------------- gradient accumulation
def test_accumulate_integer_micro_steps_exact():
    # "DeepSpeed ZeRO-3 源码解析" 5.3 / 6: micro-step 0 copies, later micro-steps
    # add into the same partition. Integer gradients keep every sum exact, so
    # the partition after M micro-steps is the int64 sum over all of them.
    rng = np.random.default_rng(21)
    K, N, M = 4, 4 * 13 + 2, 3
    steps = [rng.integers(-8, 9, size=(K, N)) for _ in range(M)]
    out = oracle.reduce_scatter([s.astype(np.float32) for s in steps[0]], N, np.float32,
                                shift=1, average=False)
    for s in steps[1:]:
        oracle.reduce_scatter([x.astype(np.float32) for x in s], N, np.float32, shift=1,
                              average=False, out=out, accumulate=True)
    total = sum(s.sum(axis=0) for s in steps)
    C = -(-N // K)
    for q in range(K):
        j = (q + 1) % K
        for o in range(C):
            g = j * C + o
            assert out[q][o] == (total[g] if g < N else 0)


@pytest.mark.parametrize("K,out_bf16", [(8, False), (8, True), (3, False), (5, True)])
def test_accumulate_is_one_add_of_old_and_average(K, out_bf16):
    import torch
    rng = np.random.default_rng(K * 2 + out_bf16)
    N = K * 40 + 3
    a = [wide_random(N, rng) for _ in range(K)]
    b = [wide_random(N, rng) for _ in range(K)]
    dt = np.uint16 if out_bf16 else np.float32
    first = oracle.reduce_scatter(a, N, dt, shift=1, average=True)
    alone = oracle.reduce_scatter(b, N, np.float32, shift=1, average=True)
    acc = [x.copy() for x in first]
    oracle.reduce_scatter(b, N, dt, shift=1, average=True, out=acc, accumulate=True)
    for q in range(K):
        if out_bf16:
            old = torch.from_numpy(first[q].view(np.int16).copy()).view(torch.bfloat16).float()
            want = (old + torch.from_numpy(alone[q])).to(torch.bfloat16).view(torch.int16)
            assert np.array_equal(acc[q], want.numpy().view(np.uint16))
        else:
            assert np.array_equal(acc[q].view(np.uint32), (first[q] + alone[q]).view(np.uint32))


def test_accumulate_into_zero_equals_plain():
    rng = np.random.default_rng(4)
    K, N = 8, 8 * 33
    xs = [wide_random(N, rng) for _ in range(K)]
    plain = oracle.reduce_scatter(xs, N, np.float32, shift=0, average=True)
    acc = [np.zeros(-(-N // K), dtype=np.float32) for _ in range(K)]
    oracle.reduce_scatter(xs, N, np.float32, shift=0, average=True, out=acc, accumulate=True)
    for q in range(K):
        # +0 + v == v for every v except -0 (which becomes +0)
        same = (plain[q] == acc[q]) & ~((plain[q] == 0) & np.signbit(plain[q]))
        assert np.all(same | ((plain[q] == 0) & (acc[q] == 0)))


# ------------------------------------------------------- bf16 wire order
def bf16_random(shape, rng):
    return oracle.bf16_to_f32(oracle.f32_to_bf16(wide_random(shape, rng)))


@pytest.mark.parametrize("K", [2, 3, 4, 7, 8, 16])
def test_wire_fold_equals_literal_bf16_ring(K):
    # a ring that carries bf16: each receiver adds in fp32 and keeps (and
    # forwards) the bf16 rounding of the new partial sum
    rng = np.random.default_rng(300 + K)
    C = 29
    x = bf16_random((K, K * C), rng)
    state, _ = oracle.ring_run(x, K - 1, 0, wire=True)
    for j in range(K):
        got = oracle.fold_points(x[:, j * C:(j + 1) * C], np.full(C, j), wire=True)
        assert np.array_equal(got.view(np.uint32), state[(j - 1) % K, j].view(np.uint32))
        # every partial that travels is a bf16 value, so the result is one too
        assert np.array_equal(got, oracle.bf16_to_f32(oracle.f32_to_bf16(got)))
    # and the all-gather phase hands everyone the same bf16 sums
    full, _ = oracle.ring_run(x, K - 1, K - 1, wire=True)
    ar = oracle.allreduce([oracle.f32_to_bf16(x[r]) for r in range(K)], K * C, wire=True)
    for r in range(K):
        assert np.array_equal(oracle.bf16_to_f32(ar[r]), full[r].reshape(-1))


def test_wire_order_handworked_ties():
    """Ranks 0..3 hold (1, d, d, d) with d = 2^-8 (bf16 keeps 8 significant bits).
    bf16 wire, by start rank (ties go to the even significand):
      start 0: 1+d ties to 1, again 1, again 1                      -> 1
      start 1: d+d = 2d, +d = 3d (exact), +1 = 1+3d ties to 1+4d   -> 1.015625
      start 2: d+d = 2d, +1 = 1+2d (exact), +d = 1+3d -> 1+4d      -> 1.015625
      start 3: d+1 ties to 1, +d -> 1, +d -> 1                      -> 1
    With fp32 accumulation every start gives 1+3d, rounded once to bf16: 1+4d."""
    d = 2.0 ** -8
    K, C = 4, 3
    vals = (1.0, d, d, d)
    ins = [oracle.f32_to_bf16(np.full(K * C, v, dtype=np.float32)) for v in vals]
    wire = oracle.reduce_scatter(ins, K * C, np.float32, shift=1, average=False, wire=True)
    ring = oracle.reduce_scatter(ins, K * C, np.uint16, shift=1, average=False)
    want_wire = (1.0, 1.015625, 1.015625, 1.0)
    for j in range(K):
        assert np.all(wire[(j - 1) % K] == np.float32(want_wire[j])), j
        assert np.all(oracle.bf16_to_f32(ring[(j - 1) % K]) == np.float32(1.015625))


def test_wire_flag_has_no_effect_on_fp32_input():
    rng = np.random.default_rng(8)
    K, N = 8, 8 * 21
    xs = [wide_random(N, rng) for _ in range(K)]
    a = oracle.reduce_scatter(xs, N, np.float32, shift=1, average=True)
    b = oracle.reduce_scatter(xs, N, np.float32, shift=1, average=True, wire=True)
    for q in range(K):
        assert np.array_equal(a[q].view(np.uint32), b[q].view(np.uint32))
