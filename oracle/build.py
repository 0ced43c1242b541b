"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

Plain gcc, -O2, no fast-math and no floating-point contraction, so every fp32
step in the oracle is one IEEE operation.  OpenMP only splits work across
output elements.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qgemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """sanitize: AddressSanitizer and UndefinedBehaviorSanitizer instrumentation
    (-O1, every finding fatal), for a checking run of the pin tests."""
    opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all"] if sanitize else ["-O2"])
    cmd = [
        "gcc", *opt, "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        SRC, "-o", out + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
