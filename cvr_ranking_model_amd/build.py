"""Build libcvr.so in-tree with hipcc for gfx950.

``python -m cvr_ranking_model_amd.build`` (or ``build()``) compiles every
``csrc/*.hip`` and ``csrc/*.cpp`` file to an object and links the shared
library next to this file.  Always recompiles.

``build(asan=True, out_dir=...)`` builds a second library, ``libcvr_asan.so`` in out_dir (a new
temporary directory by default), whose host code is compiled with AddressSanitizer (the device
code is the same as the plain build's); it is a test artefact, loaded only with the sanitizer's
runtime preloaded (``asan_runtime()``).
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcvr.so")
# host code only: every sanitizer flag goes to the host half of each hipcc compile
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(os.path.dirname(HERE), "include")]


def _hipcc():
    for c in [shutil.which("hipcc"), "/opt/rocm/bin/hipcc"]:
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def asan_runtime():
    """The shared AddressSanitizer runtime of the compiler hipcc drives (to preload)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime was not found")
    return path


def _compile(src, obj_dir, asan=False):
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, *(ASAN_FLAGS if asan else []), "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{err}")
    return obj, err


def build(verbose=False, asan=False, out_dir=None):
    if asan:
        out_dir = out_dir or tempfile.mkdtemp(prefix="cvr_asan_")
        obj_dir, lib = os.path.join(out_dir, "obj"), os.path.join(out_dir, "libcvr_asan.so")
    else:
        obj_dir, lib = OBJ, LIB
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda src: _compile(src, obj_dir, asan), srcs))
    for obj, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libcvr.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
