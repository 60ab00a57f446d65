"""Host code under the address and undefined-behaviour sanitizers.

Three builds with g++/gcc -fsanitize=address,undefined (no recovery from
undefined behaviour, so any report fails the run), each exercised by the CPU
tests of what it contains, in a child process that preloads the ASan runtime
(the Python interpreter itself is not instrumented; leak detection is off,
since the interpreter keeps its allocations until exit):
  - the oracle (oracle/oracle.c): the oracle pins;
  - the scheduler and prefetch simulators, which compile the library's own
    scheduler and prefetch cores: their replay tests;
  - the C-ABI layer (argument validation, scheduler, prefetch coordinator,
    cost model) linked with stubs for the kernel launches, which these tests
    never reach: the ABI validation and cost-model tests.
"""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1", "-fPIC", "-shared"]
CSRC = os.path.join(ROOT, "gradient_sync_zr_amd", "csrc")
KIT = os.path.join(ROOT, "tests", "kit")


def asan_runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    if shutil.which("g++") is None or asan_runtime() is None:
        pytest.skip("g++ with the ASan runtime is not available")
    d = tmp_path_factory.mktemp("san")
    out = {"oracle": str(d / "liboracle.so"), "sched": str(d / "libsched_sim.so"),
           "pf": str(d / "libpf_sim.so"), "zr": str(d / "libzr.so")}
    cmds = [
        ["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math"] + SAN +
        ["-o", out["oracle"], os.path.join(ROOT, "oracle", "oracle.c"), "-lm"],
        ["g++", "-std=c++17", "-I", CSRC] + SAN + ["-o", out["sched"], os.path.join(KIT, "sched_sim.cpp")],
        ["g++", "-std=c++17", "-I", CSRC] + SAN + ["-o", out["pf"], os.path.join(KIT, "pf_sim.cpp")],
        ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
         "-I", CSRC] + SAN + ["-o", out["zr"]] +
        [os.path.join(CSRC, f) for f in ("zr_abi.cpp", "zr_sched.cpp", "zr_prefetch.cpp", "zr_cost.cpp")] +
        [os.path.join(KIT, "host_stubs.cpp"), "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        assert r.returncode == 0, " ".join(c) + "\n" + r.stderr[-3000:]
    return out


def run_tests(files, env_extra):
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + \
          [os.path.join(ROOT, "tests", f) for f in files]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    return out


def test_oracle_pins_under_sanitizers(builds):
    run_tests(["test_oracle_pins.py"], {"ORACLE_LIBRARY": builds["oracle"]})


def test_scheduler_and_prefetch_cores_under_sanitizers(builds):
    run_tests(["test_sched_cpu.py", "test_prefetch_cpu.py"],
              {"SCHED_SIM_LIBRARY": builds["sched"], "PF_SIM_LIBRARY": builds["pf"]})


def test_abi_layer_under_sanitizers(builds):
    run_tests(["test_abi_cpu.py", "test_cost_model_cpu.py"], {"ZR_LIBRARY": builds["zr"]})
