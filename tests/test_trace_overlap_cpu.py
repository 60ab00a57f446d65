"""The trace-overlap tool of the test kit on a hand-built kernel trace, whose
unions and overlaps are worked out by hand below."""
import csv
import os
import sys

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "tests", "kit"))
import trace_overlap as T  # noqa: E402

FIELDS = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, s, e in rows:
            w.writerow({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name, "Start_Timestamp": s,
                        "End_Timestamp": e})


def test_bare_kernel_names():
    assert T.bare("void zr::(anonymous namespace)::rs_kernel<unsigned short, float, 8>(zr::A)") == "rs_kernel"
    assert T.bare("tk_delay_kernel(long long, long long, unsigned int*)") == "tk_delay_kernel"
    assert T.bare("void (anonymous namespace)::fill_kernel<0>(unsigned long)") == "fill_kernel"
    assert T.bare("rsf_kernel") == "rsf_kernel"


def test_union_and_intersection():
    assert T.union([(5, 9), (0, 3), (2, 4), (9, 12)]) == [(0, 4), (5, 12)]
    assert T.length([(0, 4), (5, 12)]) == 11
    assert T.both([(0, 4), (5, 12)], [(3, 6), (10, 20)]) == 1 + 1 + 2


def test_phases_and_hidden_fraction(tmp_path):
    us = 1000  # timestamps in ns
    rows = [
        # phase 1: reductions at [0,10) and [20,30) us, compute at [5,25) us, a copy kernel
        # of neither class at [40,60) us that must not join the two phases
        ("void zr::(anonymous namespace)::rs_kernel<unsigned short, 8>(zr::Args)", 0, 10 * us),
        ("tk_delay_kernel(long long, long long, unsigned int*)", 5 * us, 25 * us),
        ("rs_kernel", 20 * us, 30 * us), ("void (anonymous namespace)::fill_kernel<0>()", 40 * us, 60 * us),
        # phase 2, after a 1 ms gap: one reduction alone
        ("rs_kernel<x>", 1030 * us, 1040 * us),
    ]
    path = tmp_path / "trace.csv"
    write_trace(path, rows)
    ph = T.report(T.load(str(path)), ["rs_kernel"], ["tk_delay_kernel"], gap_us=200)
    assert len(ph) == 2
    p1, p2 = ph
    assert (p1["a_kernels"], p1["b_kernels"]) == (2, 1)
    assert p1["a_busy_ms"] == 0.02 and p1["b_busy_ms"] == 0.02
    assert p1["both_busy_ms"] == 0.01 and p1["a_hidden_fraction"] == 0.5
    assert p1["span_ms"] == 0.03
    assert (p2["a_kernels"], p2["b_kernels"]) == (1, 0)
    assert p2["a_hidden_fraction"] == 0.0 and p2["start_ms"] == 1.03
