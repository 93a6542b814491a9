"""Build the CPU oracle (test infrastructure): gcc, fp64, OpenMP, no fast-math."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose=False, src=None, out=None):
    """Compile the oracle (by default santa_oracle.c into liboracle.so here;
    the planted-mistake test builds altered copies elsewhere)."""
    src = src or os.path.join(HERE, "santa_oracle.c")
    out = out or os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
