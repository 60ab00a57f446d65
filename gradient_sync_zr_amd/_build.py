"""Build libzr.so (HIP, gfx950) in-tree from csrc/.

Every source is compiled with hipcc for gfx950 only, with floating-point
contraction off (so every fp32 add and multiply is one IEEE operation),
correctly rounded fp32 division, and packed-fp32 instructions disabled.
Objects go to _build/ at the repository root; the library lands next to this
file so that tests, the smoke check and the benchmark load it from the tree.

The build fails if any kernel touches private (scratch) memory: every kernel
here streams HBM from registers, and a scratch access means the compiler
spilled registers or copied the kernel-argument block to memory, which costs
bandwidth silently. The check reads each kernel's machine code (kept from the
same compile) for scratch loads and stores, and the resource remarks for VGPR
spills. A kernel may still reserve a small frame that no instruction uses:
the compiler keeps one when it parks scalar registers in vector-register
lanes (generic-K variants under high scalar pressure); that costs nothing and
is allowed.
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

# The discrete reduce-scatter's kernels compile as one unit per dtype pair
# (its largest share), so the slowest units build in parallel.
SOURCES = ["zr_rsf_bf16_f32.hip", "zr_rsf_bf16_bf16.hip", "zr_rsf_f32_f32.hip", "zr_rsf_f32_bf16.hip",
           "zr_rs.hip", "zr_ar.hip", "zr_rsf.hip", "zr_ag.hip", "zr_flatten.hip", "zr_abi.cpp", "zr_sched.cpp",
           "zr_prefetch.cpp", "zr_cost.cpp"]


_REMARK = re.compile(r"remark:\s+(Function Name: (\S+)|VGPRs Spill: (\d+))")
_SCRATCH_OP = re.compile(r"^\s+(scratch_|buffer_)(load|store)", re.M)


def spilling_kernels(remarks: str):
    """(kernel, VGPRs spilled) for every kernel the resource-usage remarks
    report with VGPR spills."""
    bad, name = [], None
    for m in _REMARK.finditer(remarks):
        if m.group(2):
            name = m.group(2)
        elif int(m.group(3)) > 0:
            bad.append((name, int(m.group(3))))
    return bad


def scratch_access_kernels(asm: str):
    """Kernels whose machine code (the device assembly of the compile) holds a
    scratch load or store."""
    bad = []
    for m in re.finditer(r"^(\S+):\s*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        if name.startswith("."):
            continue
        end = asm.find(".Lfunc_end", m.end())
        if end < 0:
            continue
        if _SCRATCH_OP.search(asm, m.end(), end):
            bad.append(name)
    return bad


def _compile(src, verbose):
    stem = os.path.splitext(src)[0]
    out = os.path.join(OBJ, stem + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".hip"):
        cmd += ["-Rpass-analysis=kernel-resource-usage", "-save-temps=obj"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=OBJ)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if src.endswith(".hip"):
        bad = spilling_kernels(r.stderr)
        if bad:
            listing = "\n".join(f"  {k}: {b} VGPRs spilled" for k, b in bad)
            raise RuntimeError(f"{src}: kernels that spill VGPRs:\n{listing}")
        asm_path = os.path.join(OBJ, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s")
        with open(asm_path) as fh:
            bad = scratch_access_kernels(fh.read())
        if bad:
            raise RuntimeError(f"{src}: kernels that access scratch memory:\n  " + "\n  ".join(bad))
        # the other temporaries are not needed
        for f in os.listdir(OBJ):
            if (f.startswith(stem + "-") or f.startswith(stem + ".hip-")) and \
                    f != os.path.basename(asm_path):
                os.remove(os.path.join(OBJ, f))
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
