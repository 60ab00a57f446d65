"""The measurement table of the design notes, rendered from the committed
rocprofv3 summaries (test kit, not part of the library).

Every `profiles/*.counters.txt` summary gives one row: the kernel and
workload (its first comment line), the average kernel time per launch (or per
step where launches vary), the achieved rate over the algorithmic bytes, and
HBM traffic over algorithmic bytes. The design notes carry this table between
the markers below, and a CPU test checks that it equals what this renders, so
the quoted figures cannot drift from the profiles.

    python tests/kit/profile_table.py            # print the table
"""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
PROFILES = os.path.join(ROOT, "profiles")
BEGIN = "<!-- profile table: rendered by tests/kit/profile_table.py -->"
END = "<!-- end of profile table -->"
PEAK_GBPS = 8000.0


def fields(path):
    kv, title = {}, None
    for line in open(path):
        line = line.rstrip("\n")
        if line.startswith("#"):
            if title is None:
                title = line.lstrip("# ").strip()
            continue
        if "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    return title, kv


def row(name):
    title, kv = fields(os.path.join(PROFILES, name))
    time_key = next((k for k in kv if k.endswith("_time_per_step_ms")), None)
    unit = "per step"
    if time_key is None:
        time_key = next(k for k in kv if k.endswith("_avg_ms"))
        unit = "per launch"
    ach_key = next(k for k in kv if k.startswith("achieved_GBps"))
    ach = float(kv[ach_key])
    ratio = kv.get("traffic_over_algorithmic", "-")
    return (f"| `{name}` | {title} | {float(kv[time_key]):.4f} ms {unit} | {ach:.1f} GB/s "
            f"({100 * ach / PEAK_GBPS:.1f}% of 8 TB/s) | {ratio} |")


def render():
    names = sorted(n for n in os.listdir(PROFILES) if n.endswith(".counters.txt"))
    lines = [BEGIN,
             "| Summary | Kernel and workload | Kernel time | Achieved (algorithmic bytes) | Traffic / algorithmic |",
             "|---|---|---|---|---|"]
    lines += [row(n) for n in names]
    lines.append(END)
    return "\n".join(lines)


def quoted(design_text):
    """The table as the design notes quote it (None when the markers are missing)."""
    m = re.search(re.escape(BEGIN) + r".*?" + re.escape(END), design_text, re.S)
    return m.group(0) if m else None


if __name__ == "__main__":
    print(render())
