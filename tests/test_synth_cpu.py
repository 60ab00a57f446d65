"""Host input generator: determinism, counter addressing and value recipes."""
import numpy as np

import synth
from synth import workloads as W


def test_counter_addressing_is_position_independent():
    a = synth.host_normal_bf16(1, 3, 0, 1000, 1e-3)
    b = synth.host_normal_bf16(1, 3, 500, 500, 1e-3)
    assert np.array_equal(a[500:], b)
    idx = np.array([999, 0, 123, 500], dtype=np.uint64)
    p = synth.host_points_normal_bf16(1, np.full(4, 3, dtype=np.uint64), idx, 1e-3)
    assert np.array_equal(p, a[idx.astype(np.int64)])
    assert not np.array_equal(a, synth.host_normal_bf16(1, 4, 0, 1000, 1e-3))
    assert not np.array_equal(a, synth.host_normal_bf16(2, 3, 0, 1000, 1e-3))


def test_splitmix_words_known_values():
    # With seed 0 and stream 0 the key is 0, so the words are the plain
    # SplitMix64 sequence started from state 0; its first outputs are the
    # published reference values of splitmix64.c seeded with 0.
    out = synth.host_words(0, 0, 0, 3)
    assert [int(x) for x in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                     0x06C45D188009454F]


def _bf16_to_f32(h):
    return (h.astype(np.uint32) << 16).view(np.float32)


def test_normal_moments_and_outliers():
    n = 400_000
    h = synth.host_normal_bf16(W.seed_of(5), 0, 0, n, 1.0, 0.01, 1e4)
    v = _bf16_to_f32(h).astype(np.float64)
    out = np.abs(v) == 9984.0   # bf16 of 1e4, rounded to nearest even
    assert abs(out.mean() - 0.01) < 0.001
    rest = v[~out]
    assert abs(rest.mean()) < 0.01 and abs(rest.std() - 1.0) < 0.01
    assert np.abs(rest).max() <= 6.0
    s = _bf16_to_f32(synth.host_normal_bf16(W.seed_of(3), 1, 0, n, 1e-3)).astype(np.float64)
    assert abs(s.std() - 1e-3) < 2e-5


def test_uniform_int_range():
    v = synth.host_uniform_int_f32(W.seed_of(1), 0, 0, 100_000, -8, 8)
    assert v.min() == -8 and v.max() == 8
    counts = np.bincount((v + 8).astype(int), minlength=17)
    assert counts.min() > 100_000 / 17 * 0.9
    b = synth.host_uniform_int_bf16(W.seed_of(1), 0, 0, 1000, -8, 8)
    assert np.array_equal(_bf16_to_f32(b), v[:1000])


def test_log_uniform_sizes():
    s = W.flatten8_numels()
    assert len(s) == 64 and min(s) >= 1 and max(s) <= 65536
    assert s == W.flatten8_numels()
    big = synth.log_uniform_sizes(7, 20000)
    lg = np.log(np.array(big, dtype=np.float64))
    # log-uniform over [1, 65537): log n roughly uniform on [0, ln 65537)
    assert abs(lg.mean() - np.log(65537) / 2) < 0.15


def test_workload_shapes():
    ps = W.llama_like_params()
    assert len(ps) == 226
    assert sum(p.numel for p in ps) == 6_738_149_376
    b = W.zero2_buckets()
    assert len(b) == 5 and b[-1] == (2_000_000_000, 376_274_560)
