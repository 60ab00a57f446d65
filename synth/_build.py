"""Build the input generators: libsynth_host.so (gcc) and libsynth_dev.so (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False):
    host_out = os.path.join(HERE, "libsynth_host.so")
    dev_out = os.path.join(HERE, "libsynth_dev.so")
    cmds = [
        ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
         "-Wall", "-o", host_out, os.path.join(HERE, "synth_host.c")],
        [HIPCC] + HIP_FLAGS + ["-o", dev_out, os.path.join(HERE, "synth_dev.hip")],
    ]
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
    return host_out, dev_out


if __name__ == "__main__":
    print(build(verbose=True))
