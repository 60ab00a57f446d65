"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case plants one mistake in a temporary copy of oracle/oracle.c (a wrong
ring send index, a reversed fold, a dropped rounding or padding rule, ...),
builds it with the oracle's own flags, and runs tests/test_oracle_pins.py
against that build in a subprocess (through ORACLE_LIBRARY). The pins must
fail for every mutant and pass for an unmodified copy. The source tree is
never modified. CPU only.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "oracle.c")

# name: (text in oracle.c, replacement). Not listed: changing the all-reduce's
# internal chunk_shift, which is an equivalent change (the reduce-scatter and
# the all-gather move chunk j to and from the same holder, and the fold still
# starts at rank j), so no output can tell it apart.
MUTANTS = {
    "ring_scatter_send_index": ("int c = phase == 0 ? mod((int64_t)r - i, K)",
                                "int c = phase == 0 ? mod((int64_t)r + i, K)"),
    "ring_gather_send_index": ("mod((int64_t)r + 1 - i, K);\n                msg_chunk",
                               "mod((int64_t)r - i, K);\n                msg_chunk"),
    "ring_wire_rounding_dropped": ("if (wire) dst[o] = orc_bf16_to_f32(orc_f32_to_bf16(dst[o]));", ""),
    "fold_first_rank": ("float acc = xs[(int64_t)s * n + p];",
                        "float acc = xs[(int64_t)((s + 1) % K) * n + p];"),
    "fold_direction": ("acc = hop(acc, xs[(int64_t)((s + h) % K) * n + p], wire);",
                       "acc = hop(acc, xs[(int64_t)((s + K - h) % K) * n + p], wire);"),
    "hop_wire_rounding_dropped": ("return wire ? orc_bf16_to_f32(orc_f32_to_bf16(acc)) : acc;",
                                  "return acc;"),
    "rs_holder": ("int j = (q + shift) % K;", "int j = (q + K - shift) % K;"),
    "rs_first_rank": ("acc = load_elem(in[j], in_dt, g);", "acc = load_elem(in[(j + 1) % K], in_dt, g);"),
    "rs_direction": ("acc = hop(acc, load_elem(in[(j + h) % K], in_dt, g), wire);",
                     "acc = hop(acc, load_elem(in[(j + K - h) % K], in_dt, g), wire);"),
    "rs_average_by_reciprocal": ("if (average) acc = acc / (float)K;",
                                 "if (average) acc = acc * (1.0f / (float)K);"),
    "rs_padding_read": ("if (g < N) {\n                acc = load_elem",
                        "if (g <= N && g < (int64_t)K * C) {\n                acc = load_elem"),
    "rs_padding_sign": ("            float acc = 0.0f;\n            if (g < N) {",
                        "            float acc = -0.0f;\n            if (g < N) {"),
    "rs_accumulate_dropped": ("if (accumulate) acc = load_elem(out[q], out_dt, o) + acc;", ""),
    "rne_ties_away": ("(lower == 0x8000u && (upper & 1u))", "(lower == 0x8000u)"),
    "rne_nan_not_quieted": ("return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)(u >> 16);"),
    "widen_low_bit": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = ((uint32_t)h << 16) | 1u;"),
    "ag_holder": ("int holder = mod((int64_t)j - shift, K);", "int holder = mod((int64_t)j + shift, K);"),
    "ag_writes_padding": ("o < C && (int64_t)j * C + o < numel", "o < C"),
    "ar_average_dropped": ("shards, shift, flags & 5);", "shards, shift, flags & 4);"),
    "flatten_offset": ("char* dst = (char*)buckets[r] + off * es;",
                       "char* dst = (char*)buckets[r] + (off + (p > 0)) * es;"),
    "flatten_padding_value": ("memset((char*)buckets[r] + off * es, 0,",
                              "memset((char*)buckets[r] + off * es, 1,"),
    "exact_sum_signed": ("a += fabs(v);", "a += v;"),
}


def run_pins(source: str, tmp: str):
    """Builds `source` and runs the pins against it; (passed, output)."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    from _build import compile_oracle
    src = os.path.join(tmp, "oracle.c")
    lib = os.path.join(tmp, "liboracle.so")
    with open(src, "w") as f:
        f.write(source)
    compile_oracle(src, lib)
    env = dict(os.environ, ORACLE_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    return r.returncode == 0, r.stdout + r.stderr


def test_every_planted_mistake_fails_a_pin():
    orig = open(SRC).read()
    jobs = {"unmodified": orig}
    for name, (a, b) in MUTANTS.items():
        assert orig.count(a) == 1, f"{name}: the text to mutate is not in oracle.c exactly once"
        jobs[name] = orig.replace(a, b)
    with tempfile.TemporaryDirectory() as top:
        def one(item):
            name, source = item
            d = os.path.join(top, name)
            os.makedirs(d)
            return name, run_pins(source, d)
        with cf.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
            results = dict(ex.map(one, jobs.items()))
    passed, out = results.pop("unmodified")
    assert passed, "the pins fail on an unmodified copy:\n" + out[-2000:]
    missed = [n for n, (ok, _) in results.items() if ok]
    assert not missed, f"mistakes no pin catches: {missed}"
    # a mutant is caught by a failing pin, or by crashing the pins' process
    # (a mutant that writes out of bounds)
    for name, (_, out) in results.items():
        assert " failed" in out or "Fatal Python error" in out, \
            f"{name}: the pins neither failed nor crashed:\n{out[-1000:]}"
