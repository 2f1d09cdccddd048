"""Build libpkv.so in-tree with hipcc for gfx950.

Usage: python -m packed_varlen_gated_amd.build   (or __graft_entry__.build()).
Always recompiles every source; objects go to _build/ and the shared library is
moved into place atomically.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")
OFFLOAD_ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={OFFLOAD_ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler away from packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # atomics stay single instructions: the compiler's wave-level rewrite of
    # a uniform-address atomic broadcasts its result at once, which makes the
    # issuing wave wait for the atomic where it is issued (the chunk kernels
    # claim their next work item a step before they use it)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def sources():
    return sorted(
        os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp"))
    )


def _compile(src, obj):
    cmd = [HIPCC] + COMMON_FLAGS + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON_FLAGS + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # host pass warns about the device-only feature flag; drop that noise
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip()]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose=True):
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(build_dir, os.path.basename(s) + ".o") for s in srcs]
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(_compile, srcs, objs))
    fd, tmp = tempfile.mkstemp(prefix="libpkv.", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = [HIPCC, f"--offload-arch={OFFLOAD_ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build()
