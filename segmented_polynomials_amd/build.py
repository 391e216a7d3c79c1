"""Build of ``libsegpoly.so`` for gfx950, in tree.

Steps: compile the host-only descriptor builder into the code generator;
run it on ``csrc/specs.txt`` to emit one HIP translation unit per registered
descriptor plus the registry; compile host sources with g++ and HIP sources
with hipcc (``--offload-arch=gfx950``, packed-FP32 instructions disabled);
link the shared library next to this file.  Every call rebuilds from
scratch; objects go to ``_build/`` (not part of the sources).

Run ``python segmented_polynomials_amd/build.py`` (it does not import the
package, whose import needs the built library) or call :func:`build`.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsegpoly.so")
BENCH_LIB = os.path.join(PKG, "libsegpoly_bench.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HOST_SOURCES = ["irreps.cpp", "cg.cpp", "tp_descriptor.cpp", "symcon_descriptor.cpp"]
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-mcode-object-version=5",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wall"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose=False, jobs=None):
    jobs = jobs or min(16, os.cpu_count() or 4)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    if os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    gen = os.path.join(BUILD, "gen")
    obj = os.path.join(BUILD, "obj")
    os.makedirs(gen)
    os.makedirs(obj)
    inc = [f"-I{CSRC}", f"-I{INCLUDE}"]

    # 1. code generator (host only)
    codegen = os.path.join(BUILD, "segpoly_codegen")
    _run(["g++", "-O2", "-std=c++17", "-Wall", *inc,
          *[os.path.join(CSRC, s) for s in HOST_SOURCES], os.path.join(CSRC, "codegen.cpp"),
          "-o", codegen], verbose)
    out = _run([codegen, os.path.join(CSRC, "specs.txt"), gen], verbose)
    gen_hip = [ln.strip() for ln in out.splitlines() if ln.strip().endswith(".hip")]

    # 2. compile
    jobs_list = []
    for s in HOST_SOURCES + ["capi.cpp", "capi_linear.cpp", "capi_sh.cpp", "capi_fctp.cpp", "capi_edge.cpp"]:
        jobs_list.append(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, s),
                          "-o", os.path.join(obj, s + ".o")])
    jobs_list.append(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(gen, "registry.cpp"),
                      "-o", os.path.join(obj, "registry.cpp.o")])
    kernels = [os.path.join(CSRC, "kernels", k) for k in ("generic.hip", "linear.hip", "sh.hip", "fctp_f32.hip", "fctp_f64.hip", "fcconv.hip", "fcconv_bwd.hip", "fctp_ps.hip", "edge_scalars.hip")]
    kernels.append(os.path.join(CSRC, "noalloc.hip"))
    for h in kernels + gen_hip:
        jobs_list.append([hipcc, *HIP_FLAGS, *inc, "-c", h,
                          "-o", os.path.join(obj, os.path.basename(h) + ".o")])
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs_list))

    # 3. link
    objs = sorted(os.path.join(obj, f) for f in os.listdir(obj))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64"], verbose)
    os.replace(tmp, LIB)

    # 4. the benchmark's traffic-replay probe: a library of its own, loaded
    # only by bench.py (the method's library does not contain it)
    probe_obj = os.path.join(BUILD, "traffic_replay.o")
    _run([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "bench", "traffic_replay.hip"), "-o", probe_obj],
         verbose)
    tmp = BENCH_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", probe_obj, "-o", tmp, f"-L{ROCM}/lib",
          "-lamdhip64"], verbose)
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
