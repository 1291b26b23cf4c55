"""Build the library with AddressSanitizer and UndefinedBehaviorSanitizer on its
host code (argument checks, tile selection, launch code), for the CPU tests.

Only the host compilation is instrumented: each sanitizer flag is passed with
-Xarch_host, so the gfx950 kernels are compiled exactly as in build.py.  The
result, libfa_mi355x_san.so, is loaded by the binding when FA_LIB_PATH names it,
with clang's ASan runtime preloaded (it carries the UBSan handlers too):

    python -m exact_attention_causal_amd.build_sanitized
    FA_LIB_PATH=$PWD/exact_attention_causal_amd/libfa_mi355x_san.so \\
    LD_PRELOAD=$(python -m exact_attention_causal_amd.build_sanitized --runtime) \\
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
    python -m pytest tests/test_abi.py tests/test_binding.py -m "not gpu"
"""
import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

from exact_attention_causal_amd import build as B

SAN_LIB = os.path.join(B.HERE, "libfa_mi355x_san.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def runtime():
    """Path of clang's ASan runtime for x86-64 hosts in this ROCm installation."""
    hits = sorted(glob.glob(os.path.join(os.path.dirname(B.HIPCC), "..", "lib", "llvm", "lib", "clang", "*",
                                         "lib", "*", "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(os.path.dirname(B.HIPCC), "..", "llvm", "lib", "clang", "*",
                                         "lib", "*", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang ASan runtime not found")
    return os.path.realpath(hits[0])


def build(verbose=False):
    tmp = tempfile.mkdtemp()

    def comp(src):
        obj = os.path.join(tmp, src + ".o")
        cmd = [B.HIPCC, *B.CFLAGS, *B.EXTRA.get(src, []), *HOST_SAN, "-c", os.path.join(B.CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(comp, B.SOURCES))
    out = SAN_LIB + ".tmp"
    subprocess.check_call([B.HIPCC, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *objs, "-o", out])
    os.replace(out, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--runtime" in sys.argv:
        print(runtime())
    else:
        print(build(verbose="-v" in sys.argv))
