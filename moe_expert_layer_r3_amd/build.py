"""Build the gfx950 HIP library in-tree: moe_expert_layer_r3_amd/libmoe_mi355x.so.

Every .hip source under csrc/ is compiled with hipcc for gfx950 only, with IEEE
fp32 division (no fast-math) and with packed-fp32 instructions disabled, then
linked into one shared library exporting the C ABI of include/moe_mi355x.h."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-ffp-contract=fast",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose=False, save_temps=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True, cwd=BUILD)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        if save_temps:
            # inspection copies (assembly, register counts) from a separate
            # compile: hipcc's -save-temps pipeline generates different code
            # (measured: expf loses an FMA contraction), so the objects that are
            # linked never come from it
            temps = os.path.join(BUILD, "temps")
            os.makedirs(temps, exist_ok=True)
            subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", os.path.join(temps, os.path.basename(obj)),
                            "-save-temps=obj"], capture_output=True, text=True, cwd=temps)
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, save_temps="--save-temps" in sys.argv))
