"""Build liboracle.so (plain C, gcc). Test infrastructure only."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def compile_oracle(src: str, out: str, verbose: bool = False) -> str:
    """Compiles one oracle source into a shared library with the oracle's flags."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", out, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out


def build(verbose: bool = False) -> str:
    return compile_oracle(os.path.join(HERE, "oracle.c"), os.path.join(HERE, "liboracle.so"), verbose)


if __name__ == "__main__":
    print(build(verbose=True))
