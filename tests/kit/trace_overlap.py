"""Overlap of two kernel classes in a rocprofv3 kernel trace (test kit, not
part of the library).

Reads a `rocprofv3 --kernel-trace -f csv` trace (Kernel_Name,
Start_Timestamp, End_Timestamp in ns). A kernel's bare name drops the return
type, namespaces, template and call arguments of the demangled name
("void zr::(anonymous namespace)::rs_kernel<...>(...)" is "rs_kernel").
Kernels whose bare names start with one of --a's prefixes form class A (say
the reductions), those starting with one of --b's prefixes class B (say the
backward compute). The timeline is cut
into phases at idle gaps longer than --gap-us, where no kernel of either
class runs (a host synchronisation between two parts of a program leaves
one). For every phase it reports:
  - each class's busy time: the union of its kernels' intervals;
  - the time both classes are busy at once;
  - the fraction of A's busy time that runs while B is busy (how much of the
    reductions a concurrent compute hides).

    python tests/kit/trace_overlap.py TRACE.csv --a rs_kernel --b tk_delay_kernel
"""
import argparse
import csv
import json
import re
import sys
from typing import List, Sequence, Tuple

Interval = Tuple[int, int]


def bare(name: str) -> str:
    """The kernel's own name inside a demangled signature."""
    s = name.replace("(anonymous namespace)::", "")
    if s.startswith("void "):
        s = s[5:]
    s = re.split(r"[<(]", s, 1)[0]
    return s.split("::")[-1].strip()


def load(path: str) -> List[Tuple[str, int, int]]:
    """(bare name, start, end) of every kernel dispatch, by start time."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((bare(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort(key=lambda x: x[1])
    return rows


def union(intervals: Sequence[Interval]) -> List[Interval]:
    """Disjoint, sorted intervals covering the same points."""
    out: List[Interval] = []
    for s, e in sorted(intervals):
        if out and s <= out[-1][1]:
            if e > out[-1][1]:
                out[-1] = (out[-1][0], e)
        else:
            out.append((s, e))
    return out


def length(merged: Sequence[Interval]) -> int:
    return sum(e - s for s, e in merged)


def both(m1: Sequence[Interval], m2: Sequence[Interval]) -> int:
    """Length of the intersection of two unions (each disjoint and sorted)."""
    i = j = 0
    tot = 0
    while i < len(m1) and j < len(m2):
        lo = max(m1[i][0], m2[j][0])
        hi = min(m1[i][1], m2[j][1])
        if hi > lo:
            tot += hi - lo
        if m1[i][1] < m2[j][1]:
            i += 1
        else:
            j += 1
    return tot


def phases(rows, gap_ns: int):
    """Groups of kernels separated by idle gaps longer than gap_ns."""
    out, cur, end = [], [], 0
    for r in rows:
        if cur and r[1] - end > gap_ns:
            out.append(cur)
            cur = []
        end = r[2] if not cur else max(end, r[2])
        cur.append(r)
    if cur:
        out.append(cur)
    return out


def report(rows, a: Sequence[str], b: Sequence[str], gap_us: float):
    pick = [r for r in rows if r[0].startswith(tuple(a)) or r[0].startswith(tuple(b))]
    res = []
    for ph in phases(pick, int(gap_us * 1000)):
        ua = union([(s, e) for n, s, e in ph if n.startswith(tuple(a))])
        ub = union([(s, e) for n, s, e in ph if n.startswith(tuple(b))])
        la, lb, lab = length(ua), length(ub), both(ua, ub)
        res.append({
            "start_ms": round((ph[0][1] - pick[0][1]) / 1e6, 3),
            "span_ms": round((max(e for _, _, e in ph) - ph[0][1]) / 1e6, 3),
            "a_kernels": sum(1 for n, _, _ in ph if n.startswith(tuple(a))),
            "b_kernels": sum(1 for n, _, _ in ph if n.startswith(tuple(b))),
            "a_busy_ms": round(la / 1e6, 3), "b_busy_ms": round(lb / 1e6, 3),
            "both_busy_ms": round(lab / 1e6, 3),
            "a_hidden_fraction": round(lab / la, 4) if la else None,
        })
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("trace")
    ap.add_argument("--a", nargs="+", required=True, help="kernel name prefixes of class A")
    ap.add_argument("--b", nargs="+", required=True, help="kernel name prefixes of class B")
    ap.add_argument("--gap-us", type=float, default=200.0)
    args = ap.parse_args(argv)
    for ph in report(load(args.trace), args.a, args.b, args.gap_us):
        print(json.dumps(ph))
    return 0


if __name__ == "__main__":
    sys.exit(main())
