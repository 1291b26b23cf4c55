"""Build the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain host C compiled with gcc and OpenMP; no HIP, no shared sources with the
GPU library.  Run as ``python oracle/build.py`` or via ``build()``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


SAN_LIB = os.path.join(HERE, "liboracle_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build liboracle.so; sanitize=True builds liboracle_san.so instead, with
    AddressSanitizer and UndefinedBehaviorSanitizer (load it with the gcc
    sanitizer runtimes preloaded; ORACLE_LIB selects it in oracle/__init__.py)."""
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    san = (["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
           if sanitize else [])
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", *san, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
