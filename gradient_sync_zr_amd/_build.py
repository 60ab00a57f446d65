"""Build libzr.so (HIP, gfx950) in-tree from csrc/.

Every source is compiled with hipcc for gfx950 only, with floating-point
contraction off (so every fp32 add and multiply is one IEEE operation),
correctly rounded fp32 division, and packed-fp32 instructions disabled.
Objects go to _build/ at the repository root; the library lands next to this
file so that tests, the smoke check and the benchmark load it from the tree.

The build fails if any kernel needs private (scratch) memory: every kernel
here streams HBM from registers, and a scratch frame means the compiler spilled
or copied the kernel-argument block to memory, which costs bandwidth silently.
"""
import concurrent.futures as cf
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "zr")
LIB = os.path.join(HERE, "libzr.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("ZR_OFFLOAD_ARCH", "gfx950")

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]

SOURCES = ["zr_rs.hip", "zr_rsf.hip", "zr_ar.hip", "zr_ag.hip", "zr_flatten.hip", "zr_abi.cpp", "zr_sched.cpp",
           "zr_prefetch.cpp", "zr_cost.cpp"]


_REMARK = re.compile(r"remark:\s+(Function Name: (\S+)|ScratchSize \[bytes/lane\]: (\d+))")


def scratch_kernels(remarks: str):
    """(kernel, bytes per lane) for every kernel the resource-usage remarks
    report with a nonzero scratch size."""
    bad, name = [], None
    for m in _REMARK.finditer(remarks):
        if m.group(2):
            name = m.group(2)
        elif int(m.group(3)) > 0:
            bad.append((name, int(m.group(3))))
    return bad


def _compile(src, verbose):
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    bad = scratch_kernels(r.stderr)
    if bad:
        listing = "\n".join(f"  {k}: {b} bytes/lane" for k, b in bad)
        raise RuntimeError(f"{src}: kernels with a scratch frame:\n{listing}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
