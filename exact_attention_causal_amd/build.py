"""Build the gfx950 HIP library (libfa_mi355x.so) in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
one shared library next to this file.  The matrix-core microbenchmark that
``bench.py --peak`` runs is built beside it as libfa_peak.so; nothing in the
attention library loads it.  Run ``python -m
exact_attention_causal_amd.build`` or call ``build()``.

``python -m exact_attention_causal_amd.build --resources [substring]`` prints
the compiler's resource report for every kernel of the device code instead
(registers, spills, LDS per workgroup and the occupancy they allow), from the
same flags; a substring keeps only the kernels whose names contain it.
"""
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfa_mi355x.so")
# the matrix-core microbenchmark (bench.py --peak), a library of its own
PEAK_LIB = os.path.join(HERE, "libfa_peak.so")
PEAK_SOURCE = "peak.hip"
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_merge.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results go straight to VGPRs (no AGPR round trips for the
    # softmax and rescale work done on the accumulators)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-ffp-contract=fast", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file scheduler choice: the backward kernels measured ~0.5 % faster when
# the pre-RA scheduler groups memory operations (no effect on results).
EXTRA = {"fa_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    tmp = PEAK_LIB + ".tmp"
    cmd = [HIPCC, *CFLAGS, "-shared", os.path.join(CSRC, PEAK_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PEAK_SOURCE}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PEAK_LIB)
    return LIB


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)")


def kernel_label(sym: str) -> str:
    """Readable name of one of this library's kernel symbols, e.g.
    ``fwd_kernel<bf16, FwdTile<bf16, 128, 2, 32, 8, 1>, bf16, false>`` (the
    function parameters are left out).  Template arguments are bf16 and float
    types, integer and bool literals and class templates of namespace fa;
    anything else returns the symbol as it is."""

    def name(i):  # <length><identifier>
        m = re.match(r"\d+", sym[i:])
        n = int(m.group(0))
        return sym[i + m.end():i + m.end() + n], i + m.end() + n

    def args(i):  # I arg... E
        out = []
        i += 1
        while sym[i] != "E":
            if sym.startswith("DF16b", i):
                out.append("bf16"); i += 5
            elif sym[i] == "f":
                out.append("float"); i += 1
            elif sym[i] == "L":
                m = re.match(r"L([ib])(n?)(\d+)E", sym[i:])
                v = ("-" if m.group(2) else "") + m.group(3)
                out.append(v if m.group(1) == "i" else ("true" if v == "1" else "false")); i += m.end()
            elif sym.startswith("NS_", i):  # fa::Name<...> (nested name closed by a second E)
                n, i = name(i + 3)
                inner, i = args(i)
                out.append(f"{n}<{', '.join(inner)}>")
                if sym[i] != "E":
                    raise ValueError(sym)
                i += 1
            else:
                raise ValueError(sym)
        return out, i + 1

    try:
        if not sym.startswith("_ZN2fa"):
            return sym
        n, i = name(6)
        if i < len(sym) and sym[i] == "I":
            a, _ = args(i)
            return f"{n}<{', '.join(a)}>"
        return n
    except (ValueError, AttributeError, IndexError):
        return sym


def resources(pattern: str = ""):
    """Per-kernel resource usage as the compiler reports it for these flags.

    Returns dicts with the mangled and demangled name, VGPRs, AGPRs, spilled
    registers, scratch bytes per lane, LDS bytes per workgroup and the waves
    per SIMD (of 8) that registers and LDS allow.
    """
    rows = []
    with tempfile.TemporaryDirectory() as tmp:
        for src in SOURCES:
            cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage",
                   "-c", os.path.join(CSRC, src), "-o", os.path.join(tmp, src + ".o")]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
            for line in r.stderr.splitlines():
                m = _REMARK.search(line)
                if not m:
                    continue
                key, val = m.groups()
                if key == "Function Name":
                    rows.append({"symbol": val, "source": src})
                elif rows:
                    rows[-1][key] = int(val)
    out = []
    for r in rows:
        d = kernel_label(r["symbol"])
        if pattern and pattern not in d and pattern not in r["symbol"]:
            continue
        out.append({"symbol": r["symbol"], "name": d, "source": r["source"], "vgprs": r.get("VGPRs"),
                    "agprs": r.get("AGPRs"), "spills": r.get("VGPRs Spill", 0) + r.get("SGPRs Spill", 0),
                    "scratch": r.get("ScratchSize [bytes/lane]"), "lds": r.get("LDS Size [bytes/block]"),
                    "waves_per_simd": r.get("Occupancy [waves/SIMD]")})
    return out


if __name__ == "__main__":
    if "--resources" in sys.argv:
        rest = [a for a in sys.argv[1:] if a != "--resources"]
        print("waves/SIMD  VGPRs  AGPRs  spills  scratch  LDS bytes  kernel")
        for r in resources(rest[0] if rest else ""):
            print(f"{r['waves_per_simd']:>10}  {r['vgprs']:>5}  {r['agprs']:>5}  {r['spills']:>6}  {r['scratch']:>7}  "
                  f"{r['lds']:>9}  {r['name']}")
    else:
        print(build(verbose="-v" in sys.argv))
