"""Host-sanitized build of the C ABI: libls_mi355_san.so, whose host code
(argument validation, launch-shape tables, error bookkeeping) is compiled
with AddressSanitizer and UndefinedBehaviorSanitizer.  The device code is
compiled exactly as in the product build; only the host pass is instrumented.

Used by the CPU test that runs the ABI checks against it (the GPU is never
touched: every call there fails validation or launches nothing).
Usage: python -m non_gemm_amd.build_sanitized [OUT_DIR]
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from non_gemm_amd import build as B

# Sanitizers for the host pass only (the option after each -Xarch_host).
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime():
    """The clang ASan runtime that a non-instrumented python must preload."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found under /opt/rocm/lib/llvm")
    return hits[-1]


def _compile(src, obj_dir):
    obj = os.path.join(obj_dir, os.path.basename(src)[:-4] + ".o")
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN
    r = subprocess.run([B.hipcc(), *flags, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{B.diagnostics(r.stdout + r.stderr)}")
    return obj


def build(out_dir):
    """Builds into out_dir (outside the repository: the instrumented library
    is a test artefact) and returns the library's path."""
    obj_dir = os.path.join(out_dir, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    lib_path = os.path.join(out_dir, "libls_mi355_san.so")
    srcs = B.sources()
    with ThreadPoolExecutor(max(1, min(len(srcs), 8))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), srcs))
    tmp = lib_path + ".tmp"
    r = subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan",
                        *HOST_SAN, *objs, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    import tempfile
    print("built", build(sys.argv[1] if len(sys.argv) > 1 else tempfile.mkdtemp(prefix="ls_mi355_san_")))
    sys.exit(0)
