"""Build the HIP library ``libkvreloc.so`` in-tree for gfx950.

``python rope_rotation_splice_amd/build.py`` (or ``build()``) compiles every
source under ``csrc/`` with hipcc and links the shared library next to this
file.  It always recompiles.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkvreloc.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the device code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source additions.  band.hip: its kernel's leading scalar arguments are
# preloaded into scalar registers at launch (gfx950 kernarg preloading; the
# compiler also emits the fallback that loads them itself).
SOURCE_FLAGS = {
    "band.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
}


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose=False):
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT, flush=True)
    return OUT


SANITIZED = os.path.join(BUILD_DIR, "sanitized", "libkvreloc.so")


def build_sanitized(verbose=False):
    """A copy of the library whose host code (api.cpp: validation, planning,
    launches) is built with AddressSanitizer and UndefinedBehaviorSanitizer;
    the device objects of the last build() are linked in unchanged.  Load it
    with the sanitizer runtime preloaded (see sanitizer_runtime())."""
    hipcc = _hipcc()
    out_dir = os.path.dirname(SANITIZED)
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = os.path.join(out_dir, "api.cpp.o")
    cmds = [[hipcc, *FLAGS, "-g", *san, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj]]
    dev = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in sources() if not s.endswith("api.cpp")]
    if not all(os.path.exists(o) for o in dev):
        build(verbose)                   # the device objects come from the regular build
    objs = [api_obj] + dev
    cmds.append([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, *objs, "-o", SANITIZED])
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build failed:\n{r.stdout}\n{r.stderr}")
    return SANITIZED


def sanitizer_runtime():
    """Path of the AddressSanitizer runtime of the compiler that built the
    sanitized library (to preload into the process that loads it)."""
    hipcc = _hipcc()
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(c):
            r = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            p = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
                return p
    raise RuntimeError("AddressSanitizer runtime not found")


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        build(verbose="-v" in sys.argv)
