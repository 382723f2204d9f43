"""Build libls_mi355.so (in-tree) from the HIP sources in csrc/ for gfx950.

Usage: python -m non_gemm_amd.build   (or __graft_entry__.build()).
Every call recompiles.  hipcc cross-compiles for gfx950 without a GPU.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libls_mi355.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 VALU forms are kept out of the generated device code.  The
    # host pass receives the same cc1 option and prints HOST_FEATURE_NOTE for
    # it (the driver cannot forward cc1 options to the device pass alone);
    # _compile() drops exactly that line and shows every other diagnostic.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ls_mi355 library needs ROCm's hipcc")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def diagnostics(text):
    """Compiler output without the host pass's note about the device-only feature."""
    return "\n".join(l for l in text.splitlines() if l.strip() and l.strip() != HOST_FEATURE_NOTE)


def _compile(src):
    obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{diagnostics(r.stderr)}")
    msg = diagnostics(r.stdout + "\n" + r.stderr)
    if msg:
        print(f"{os.path.basename(src)}:\n{msg}", file=sys.stderr)
    return obj


def build(verbose=False):
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    workers = max(1, min(len(srcs), 8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
