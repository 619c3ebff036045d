"""Compile the CPU oracle (plain C, OpenMP) into oracle/liboracle.so.

Test infrastructure: the oracle is a checker, never part of the product path.
build(sanitize=True) makes an AddressSanitizer + UndefinedBehaviorSanitizer
build of the same source instead (_build/sanitize/liboracle.so), which the
sanitizer test loads through ISG_ORACLE_LIB.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "isg_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(os.path.dirname(HERE), "_build", "sanitize", "liboracle.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"])
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = ["gcc"] + opt + ["-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
                           SRC, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
