"""Build libpagedattn.so for gfx950 in-tree.

The HIP sources are compiled with hipcc for gfx950 only; the host-only block
manager and scheduler are compiled with g++.  Objects go to _build/ next to
this file and the shared library to this package directory, where the
binding loads it.

build(sanitize=True) additionally builds libpagedattn_san.so, a copy of the
library whose host code -- the C ABI's validation (api.hip), the block
manager and the scheduler -- is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (clang's runtimes; the device kernels are the
unchanged objects of the normal build, and no device code is instrumented).
The CPU tests load it with the ASan runtime preloaded (see
tests/test_sanitized_host.py); it is a checking build, never the product.

build(debug=True) additionally builds libpagedattn_debug.so: every HIP source
compiled with -DPA_DEBUG, so that the kernels count the device metadata
(block ids, context lengths, slots, copy pairs) they clamp or skip, read back
with pa_debug_counters.  Also a checking build, loaded through PAGEDATTN_LIB.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
BUILD_SAN = os.path.join(HERE, "_build_san")
BUILD_DEBUG = os.path.join(HERE, "_build_debug")
LIB = os.path.join(HERE, "libpagedattn.so")
LIB_SAN = os.path.join(HERE, "libpagedattn_san.so")
LIB_DEBUG = os.path.join(HERE, "libpagedattn_debug.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE]
SAN = ["address", "undefined"]
# host-side instrumentation only: every sanitizer flag of a hipcc line is
# bound to the host compilation
HIP_SAN_FLAGS = [f for s in SAN for f in ("-Xarch_host", f"-fsanitize={s}")] + [
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-O1"]
CXX_SAN_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
# the host sources the sanitized build instruments (the rest of the library
# is kernels and their launch wrappers)
SAN_HIP = ("api.hip",)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the fp32 packing feature; that note is harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)


def asan_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (to preload)."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, jobs: int | None = None, sanitize: bool = True, debug: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hip_srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp_srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    cmds, objs = [], []
    for f in hip_srcs:
        o = os.path.join(BUILD, f + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    for f in cpp_srcs:
        o = os.path.join(BUILD, f + ".o")
        cmds.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    san_objs = []
    if sanitize:
        os.makedirs(BUILD_SAN, exist_ok=True)
        for f in SAN_HIP:
            o = os.path.join(BUILD_SAN, f + ".o")
            cmds.append([HIPCC, *HIP_FLAGS, *HIP_SAN_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
            san_objs.append(o)
        for f in cpp_srcs:
            o = os.path.join(BUILD_SAN, f + ".o")
            cmds.append([CLANGXX, *CXX_SAN_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
            san_objs.append(o)
    debug_objs = []
    if debug:
        os.makedirs(BUILD_DEBUG, exist_ok=True)
        for f in hip_srcs:
            o = os.path.join(BUILD_DEBUG, f + ".o")
            cmds.append([HIPCC, *HIP_FLAGS, "-DPA_DEBUG", "-c", os.path.join(CSRC, f), "-o", o])
            debug_objs.append(o)
    jobs = jobs or min(8, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _link(objs, LIB, verbose)
    if sanitize:
        plain = [o for o in objs if not any(os.path.basename(o).startswith(f) for f in SAN_HIP + tuple(cpp_srcs))]
        _link(plain + san_objs, LIB_SAN, verbose)
    if debug:
        _link(debug_objs + [o for o in objs if o.endswith(".cpp.o")], LIB_DEBUG, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
