"""Build the CPU oracle library (test infrastructure only).

Compiles ggq_oracle.c with gcc into oracle/libggq_oracle.so.  Plain C,
no fast-math, no fp contraction, OpenMP over independent output rows.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ggq_oracle.c")
LIB = os.path.join(HERE, "libggq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_sanitized(out: str) -> str:
    """The same source with gcc's AddressSanitizer and UndefinedBehaviorSanitizer
    (host code only: the oracle is plain C).  Load it into a process that
    preloads gcc's libasan and libubsan."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-o", out, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
