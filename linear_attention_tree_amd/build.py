"""Build libbole.so (HIP, gfx950) in-tree.

Every .hip file under csrc/ is compiled to an object in parallel, then linked
into linear_attention_tree_amd/libbole.so; the measurement baselines under
baselines/ go into baselines/libbole_baselines.so.  hipcc cross-compiles for
gfx950 without a GPU present.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libbole.so")
# measurement baselines (not part of libbole's interface)
BASELINE_DIR = os.path.join(HERE, "baselines")
BASELINE_LIB_PATH = os.path.join(BASELINE_DIR, "libbole_baselines.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=fast",
    # packed fp32 instructions stay off for the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libbole")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Build libbole.so and the measurement baselines' library; returns the
    path of libbole.so."""
    path = _build_lib(sources(), LIB_PATH, "", verbose, jobs)
    _build_lib(sorted(glob.glob(os.path.join(BASELINE_DIR, "*.hip"))), BASELINE_LIB_PATH,
               "baseline_", verbose, jobs)
    return path


def _build_lib(srcs, lib_path, prefix, verbose, jobs):
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(BUILD_DIR, prefix + os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out, file=sys.stderr)

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = lib_path + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
