"""Build the HIP shared libraries in-tree for gfx950.

  collective_communication_reduction_amd/libgc.so   the collectives (C ABI in include/gc.h)
  gen/libgcgen.so                                   device twin of the input generator
  tests/abi_c/abi_demo                              a plain C program using libgc through gc.h alone
  libbenchpatterns.so                               access-pattern ceilings for bench.py --patterns

Usage: python collective_communication_reduction_amd/build.py  (or build() from Python).
Every call recompiles; hipcc cross-compiles without a GPU.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"

# Floating-point flags the results depend on: no contraction of a*b+c into an
# FMA, correctly rounded fp32 division, fp32 subnormals kept.  Packed fp32
# instructions are switched off for the device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

LIB_SOURCES = ["api.cpp", "reduce.hip", "movement.hip", "bucket.hip", "moe.hip", "hier.hip"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in p.stderr.splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _compile(hipcc, src, obj, includes, verbose):
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc] + HIP_FLAGS + [f"-I{d}" for d in includes] + lang + ["-c", src, "-o", obj]
    _run(cmd, verbose)
    return obj


def build(verbose=False):
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    includes = [os.path.join(ROOT, "include"), CSRC]
    jobs = []
    for s in LIB_SOURCES:
        jobs.append((os.path.join(CSRC, s), os.path.join(BUILD, s + ".o")))
    gen_src = os.path.join(ROOT, "gen", "device.hip")
    gen_obj = os.path.join(BUILD, "gen_device.o")
    jobs.append((gen_src, gen_obj))
    pat_src = os.path.join(ROOT, "bench_patterns.hip")
    pat_obj = os.path.join(BUILD, "bench_patterns.o")
    jobs.append((pat_src, pat_obj))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda j: _compile(hipcc, j[0], j[1], includes, verbose), jobs))
    lib = os.path.join(PKG, "libgc.so")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", lib + ".tmp"]
         + [o for s, o in jobs if s not in (gen_src, pat_src)], verbose)
    os.replace(lib + ".tmp", lib)
    genlib = os.path.join(ROOT, "gen", "libgcgen.so")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", genlib + ".tmp", gen_obj], verbose)
    os.replace(genlib + ".tmp", genlib)
    patlib = os.path.join(ROOT, "libbenchpatterns.so")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", patlib + ".tmp", pat_obj], verbose)
    os.replace(patlib + ".tmp", patlib)
    demo = build_c_demo(verbose)
    return lib, genlib, patlib, demo


def build_c_demo(verbose=False):
    """The C consumer of the ABI, compiled as C11 by the host C compiler (gc.h is a
    C header) and linked against libgc.so and the HIP runtime."""
    src = os.path.join(ROOT, "tests", "abi_c", "abi_demo.c")
    out = os.path.join(ROOT, "tests", "abi_c", "abi_demo")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for tests/abi_c/abi_demo.c")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    _run([cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
          f"-I{os.path.join(ROOT, 'include')}", "-isystem", os.path.join(rocm, 'include'), src, "-o", out + ".tmp",
          f"-L{PKG}", "-lgc", f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/../../collective_communication_reduction_amd", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"],
         verbose)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    for path in build(verbose="-v" in sys.argv):
        print(path)
