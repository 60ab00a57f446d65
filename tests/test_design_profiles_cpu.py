"""The design notes quote the committed profiles exactly: the measurement
table between its markers in the design doc equals the one rendered from
profiles/*.counters.txt, so a re-taken profile without an updated table (or
a hand-edited figure) fails here."""
import os
import sys

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "tests", "kit"))
import profile_table  # noqa: E402


def test_design_table_equals_the_profiles():
    design = open(os.path.join(ROOT, "DESIGN.md")).read()
    got = profile_table.quoted(design)
    assert got is not None, "DESIGN.md has no profile table"
    assert got == profile_table.render(), "run tests/kit/profile_table.py and paste its output"


def test_every_counter_summary_renders_a_row():
    rendered = profile_table.render()
    names = [n for n in os.listdir(profile_table.PROFILES) if n.endswith(".counters.txt")]
    assert len(names) >= 5
    for n in names:
        assert f"`{n}`" in rendered
