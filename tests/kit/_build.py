"""Build the test kit: libsched_sim.so and libpf_sim.so (g++), libtestkit.so (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False):
    cmds = [
        ["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-I", os.path.join(ROOT, "gradient_sync_zr_amd", "csrc"),
         "-o", os.path.join(HERE, "libsched_sim.so"), os.path.join(HERE, "sched_sim.cpp")],
        ["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-I", os.path.join(ROOT, "gradient_sync_zr_amd", "csrc"),
         "-o", os.path.join(HERE, "libpf_sim.so"), os.path.join(HERE, "pf_sim.cpp")],
        [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", os.path.join(HERE, "libtestkit.so"), os.path.join(HERE, "testkit.hip")],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


if __name__ == "__main__":
    build(verbose=True)
