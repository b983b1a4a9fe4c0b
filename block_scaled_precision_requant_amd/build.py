"""Build libbsr.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source is compiled by hipcc with IEEE float semantics (no fast-math, no
FMA contraction unless written, subnormals kept) and without packed-FP32
instructions, then linked into block_scaled_precision_requant_amd/libbsr.so.
Symbols are hidden by default: the library exports exactly the functions
include/bsr.h declares (marked BSR_API there).
"""
import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsr.so")
SOURCES = ["requant.hip", "gemm.hip", "gemv.hip", "w4a16.hip", "api.hip"]
# The streaming-read kernel bench.py reports as bandwidth context: a library of
# its own, so libbsr.so exports only the entry points include/bsr.h declares.
READ_LIB = os.path.join(PKG, "libbsr_read.so")
READ_SOURCE = "read_probe.hip"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source additions: the GEMV kernels' matrix-core results are consumed by
# vector FP32 code, so they must land in ordinary VGPRs (the default heuristic
# puts them in AGPRs for one-wave workgroups, costing a copy per value).
EXTRA_FLAGS = {"gemv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, save_temps):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if save_temps:
        cmd.insert(1, f"-save-temps={'obj'}")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def declared_functions():
    """Names of the functions include/bsr.h declares (each marked BSR_API)."""
    with open(os.path.join(INCLUDE, "bsr.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(re.findall(r"^BSR_API\s+(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def _version_script():
    """Linker version script: the declared functions global, every other symbol
    (the compiler's per-unit HIP identifiers included) local."""
    path = os.path.join(BUILD, "libbsr.map")
    body = "".join(f"    {name};\n" for name in declared_functions())
    with open(path, "w") as f:
        f.write("{\n  global:\n" + body + "  local: *;\n};\n")
    return path


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile every kernel source and link libbsr.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES + [READ_SOURCE]))
    read_obj = objs.pop()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
           f"-Wl,--version-script={_version_script()}", "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    tmp = READ_LIB + ".tmp%d" % os.getpid()
    read_map = os.path.join(BUILD, "libbsr_read.map")
    with open(read_map, "w") as f:
        f.write("{\n  global:\n    read_probe;\n  local: *;\n};\n")
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", read_obj,
                    f"-Wl,--version-script={read_map}", "-o", tmp], check=True, capture_output=not verbose)
    os.replace(tmp, READ_LIB)
    if verbose:
        print(LIB, READ_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
